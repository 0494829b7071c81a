"""Plain float64 definitions of the sparse-MLA hot path.

Test infrastructure only (see the package header). Notation: T query tokens, H heads,
W entries per index list, P page size, 576 = 512 latent + 64 rotary columns per row,
tau the softmax scale.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, f32_to_bf16_rne, e4m3_decode, e4m3_encode, E4M3_MAX

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE
ROW_BITS = 24            # union entries keep the row in bits 0..23, membership above
INT32_MAX = 2 ** 31 - 1  # slots are 32-bit integers

KV_F32 = "f32"
KV_BF16 = "bf16"
KV_FP8 = "fp8"


# ----------------------------------------------------------------------------------
# Slot resolution
# ----------------------------------------------------------------------------------

def resolve_slots(idx, valid, tok_req, page_table, seq_lens, page_size):
    """Physical cache slot of every logical index.

    A paged kernel maps position `pos` of request `req` to
    page_table[req, pos // P] * P + pos % P (The Virtual Block Table, "The
    Investigation"); with P = 1 this is page_table[req, pos] itself ("Assumptions and
    Reasoning", Assumption 1), which is how request-relative top-k indices become global
    slots before the decode kernel sees them.

    An entry resolves to -1 when it is padding or out of range: j >= valid[t] (the
    per-token count of valid entries), a token whose request is not a row of the page
    table, a negative index, an index at or past the request's context length, past the
    page-table row, on a page whose id is < 0, or when the slot itself is past 2^31 - 1
    (slots are 32-bit integers, so no pool has such a row).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, W = idx.shape
    pt = np.asarray(page_table, dtype=np.int64)
    req_raw = np.asarray(tok_req, dtype=np.int64)[:, None]
    req_ok = (req_raw >= 0) & (req_raw < pt.shape[0])
    req = np.where(req_ok, req_raw, 0)
    j = np.arange(W)[None, :]
    n = W if valid is None else np.asarray(valid, dtype=np.int64)[:, None]
    ok = req_ok & (j < n) & (idx >= 0) & (idx < np.asarray(seq_lens, dtype=np.int64)[req])
    page_no = np.where(ok, idx // page_size, 0)
    ok &= page_no < pt.shape[1]
    page = pt[req, np.minimum(page_no, pt.shape[1] - 1)]
    ok &= page >= 0
    slot = page * page_size + idx % page_size
    ok &= slot <= INT32_MAX                  # a slot no int32 table can name (reading: masked)
    return np.where(ok, slot, -1).astype(np.int32)


def attended_slots(table_row, length, page_size):
    """The slots one query token attends to, in table order.

    Page size 1 (the virtual block table, "The Breakthrough"): the first `length`
    entries of the row are slots; entries < 0 are padding and skipped.
    Page size P > 1 (the dense paged case): positions 0..length-1 through the row's
    page ids; positions past the row or on a page id < 0 are skipped.
    """
    row = np.asarray(table_row, dtype=np.int64)
    n = max(int(length), 0)
    if page_size == 1:
        sel = row[:min(n, len(row))]
        return sel[sel >= 0]
    p = np.arange(n, dtype=np.int64)
    p = p[p // page_size < len(row)]
    page = row[p // page_size]
    keep = page >= 0
    return page[keep] * page_size + p[keep] % page_size


# ----------------------------------------------------------------------------------
# The latent KV pool and the cache write
# ----------------------------------------------------------------------------------

class Pool:
    """A pool of `num_slots` latent rows, held sparsely; never-written slots read as NaN.

    dtype "f32"/"bf16": one stored row of 576 values per slot.
    dtype "fp8": e4m3 codes for the 512 latent values, the 64 rotary values in bf16 and
    one float32 scale per slot; the row's value is code * scale for the latent part.
    """

    def __init__(self, num_slots: int, dtype: str):
        assert dtype in (KV_F32, KV_BF16, KV_FP8)
        self.num_slots = int(num_slots)
        self.dtype = dtype
        self.slots = np.zeros(0, np.int64)
        if dtype == KV_F32:
            self.planes = {"rows": np.zeros((0, ROW), np.float32)}
        elif dtype == KV_BF16:
            self.planes = {"rows": np.zeros((0, ROW), np.uint16)}
        else:
            self.planes = {"lat8": np.zeros((0, LATENT), np.uint8),
                           "rope16": np.zeros((0, ROPE), np.uint16),
                           "scale": np.zeros(0, np.float32)}

    def store(self, slots, planes):
        """Overwrite the stored planes of the given (distinct, in-range) slots."""
        slots = np.asarray(slots, dtype=np.int64)
        assert len(np.unique(slots)) == len(slots)
        assert np.all((slots >= 0) & (slots < self.num_slots))
        keep = ~np.isin(self.slots, slots)
        merged = np.concatenate([self.slots[keep], slots])
        order = np.argsort(merged, kind="stable")
        self.slots = merged[order]
        for k in self.planes:
            self.planes[k] = np.concatenate([self.planes[k][keep], planes[k]])[order]

    def stored(self, slots):
        """The stored planes of the given slots (must have been written)."""
        pos = np.searchsorted(self.slots, slots)
        assert np.all(self.slots[np.minimum(pos, len(self.slots) - 1)] == slots)
        return {k: v[pos] for k, v in self.planes.items()}

    def rows(self, slots):
        """Value of each requested row as float64 [n, 576]; NaN rows for unwritten slots."""
        slots = np.asarray(slots, dtype=np.int64)
        out = np.full((len(slots), ROW), np.nan)
        if len(self.slots) == 0 or len(slots) == 0:
            return out
        pos = np.minimum(np.searchsorted(self.slots, slots), len(self.slots) - 1)
        hit = self.slots[pos] == slots
        p = pos[hit]
        if self.dtype == KV_F32:
            out[hit] = self.planes["rows"][p].astype(np.float64)
        elif self.dtype == KV_BF16:
            out[hit] = bf16_bits_to_f64(self.planes["rows"][p])
        else:
            sc = self.planes["scale"][p].astype(np.float64)[:, None]
            out[hit, :LATENT] = e4m3_decode(self.planes["lat8"][p]) * sc
            out[hit, LATENT:] = bf16_bits_to_f64(self.planes["rope16"][p])
        return out


def kv_write(pool: Pool, src, src_dtype: str, slot_mapping):
    """Write token rows into their cache slots (the KV write that precedes attention in a
    decode step: The Assertion That Changed Everything, "The Message").

    src: [n, 576] float32 values (src_dtype "f32") or bf16 bit patterns ("bf16").
    slot_mapping[i] < 0 skips row i.

    Stored form by cache dtype:
      f32  -- the float32 value (bf16 sources are exact in float32);
      bf16 -- nearest bf16 of the float32 value, ties to even;
      fp8  -- amax = max |c| over the 512 latent values (float32), scale = amax / 448
              rounded to float32, code = e4m3 of the float32 quotient c / scale (nearest,
              ties to even, saturating at 448), all codes 0 when scale is 0; the 64
              rotary values as bf16 (nearest, ties to even); the scale as float32.
    """
    src = np.asarray(src)
    if src_dtype == KV_BF16:
        x32 = (src.astype(np.uint32) << 16).view(np.float32)
    else:
        x32 = src.astype(np.float32)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    live = sm >= 0
    x32 = x32[live]
    slots = sm[live]
    if pool.dtype == KV_F32:
        pool.store(slots, {"rows": x32.copy()})
    elif pool.dtype == KV_BF16:
        pool.store(slots, {"rows": f32_to_bf16_rne(x32)})
    else:
        lat = x32[:, :LATENT]
        amax = np.max(np.abs(lat), axis=1).astype(np.float32)
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            quot = (lat / scale[:, None]).astype(np.float32)
        codes = e4m3_encode(quot)
        codes[scale == 0] = 0
        pool.store(slots, {"lat8": codes, "rope16": f32_to_bf16_rne(x32[:, LATENT:]),
                           "scale": scale})


# ----------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------

def attention(qh, rows, scale):
    """Softmax attention of H query heads over n gathered rows.

    qh: [H, 576] float64; rows: [n, 576] float64. Every head's score against a row is
    tau times the full 576-wide dot product (latent part against the absorbed q_nope,
    rotary part against q_rope); the value is the first 512 columns of the same row, so
    the output is 512 wide (vLLM PR 63104, bench_shardq_rank.py: the q split into
    [:LORA] and [LORA:] parts and the 512-wide output; The Virtual Block Table,
    "Assumptions and Reasoning", Assumption 2: K and V are views of one cache).

    Returns O [H, 512] and LSE [H] = natural log of sum_j exp(s_hj). No rows gives
    O = 0 and LSE = -inf.
    """
    H = qh.shape[0]
    n = rows.shape[0]
    if n == 0:
        return np.zeros((H, LATENT)), np.full(H, -np.inf)
    s = scale * (qh @ rows.T)                       # [H, n]
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    lse = m + np.log(z)
    p = np.exp(s - lse)                             # softmax weights
    o = p @ rows[:, :LATENT]
    return o, lse[:, 0]


def _q_f64(q, q_dtype):
    q = np.asarray(q)
    return bf16_bits_to_f64(q) if q_dtype == KV_BF16 else q.astype(np.float64)


def sparse_decode(q, q_dtype, pool: Pool, table, lens, page_size, scale, tokens=None):
    """Decode attention of every query token over its attended slots.

    page_size 1: `table` rows are resolved top-k slots and `lens` the valid counts (the
    virtual block table, The Virtual Block Table, "The Breakthrough"); page_size P > 1:
    `table` rows are page ids and `lens` context lengths (the paged decode the same
    interface was built for).

    q: [T, H, 576] float32 or bf16 bits. Returns O [T', H, 512], LSE [T', H] float64 for
    the tokens listed in `tokens` (default: all).
    """
    q = np.asarray(q)
    T, H = q.shape[0], q.shape[1]
    tokens = range(T) if tokens is None else tokens
    outs, lses = [], []
    for t in tokens:
        sl = attended_slots(table[t], lens[t], page_size)
        o, l = attention(_q_f64(q[t], q_dtype), pool.rows(sl), scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def lse_combine(outs, lses):
    """Merge partial results over disjoint row sets: LSE = log sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s (IBM Triton paged-attention explainer, section 4 table,
    "Parallel Tiled Softmax"). Parts with LSE_s = -inf (no rows) contribute nothing."""
    lses = np.asarray(lses)                          # [S, H]
    outs = np.asarray(outs)                          # [S, H, 512]
    m = np.max(lses, axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - msafe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.einsum("sh,shd->hd", np.where(finite, w / np.where(finite, tot, 1.0), 0.0), outs)
    return o, lse


def split_attention(qh, rows, scale, num_splits):
    """Attention computed on `num_splits` contiguous chunks of the rows (some possibly
    empty) and merged with lse_combine; equal to `attention` in exact arithmetic."""
    n = rows.shape[0]
    bounds = np.linspace(0, n, num_splits + 1).round().astype(int)
    parts = [attention(qh, rows[bounds[s]:bounds[s + 1]], scale) for s in range(num_splits)]
    return lse_combine([p[0] for p in parts], [p[1] for p in parts])


# ----------------------------------------------------------------------------------
# Grouped prefill
# ----------------------------------------------------------------------------------

def group_union(slots, valid, G, num_slots):
    """Top-k union of each group of G consecutive queries, with membership bits.

    Group g holds queries gG .. min(gG+G, Q)-1 (the last group may be short). Its union
    is the ascending set of rows r with 0 <= r < num_slots that some member lists within
    its first valid[q] entries; entry = r | (mask << 24), where bit i of mask says that
    member i lists r (vLLM PR 63104, "Tests": rows past a query's count and negative
    rows are ignored, rows reach the 24-bit limit; "Changes": the mask keeps each query
    to its own top-k; "Details": one membership mask per query).

    Returns enc uint32 [ceil(Q/G), G*W] (entries past lens[g] are 0 here; the library
    leaves them unspecified) and lens int32 [ceil(Q/G)].
    """
    slots = np.asarray(slots, dtype=np.int64)
    Q, W = slots.shape
    ng = -(-Q // G)
    enc = np.zeros((ng, G * W), dtype=np.uint32)
    lens = np.zeros(ng, dtype=np.int32)
    for g in range(ng):
        lists = []
        for i in range(G):
            qi = g * G + i
            if qi >= Q:
                lists.append(np.zeros(0, np.int64))
                continue
            lst = slots[qi, :min(max(int(valid[qi]), 0), W)]
            lists.append(lst[(lst >= 0) & (lst < num_slots)])
        union = np.unique(np.concatenate(lists))      # ascending, distinct
        mask = np.zeros(len(union), np.int64)
        for i, lst in enumerate(lists):
            mask |= np.isin(union, lst).astype(np.int64) << i
        enc[g, :len(union)] = (union | (mask << ROW_BITS)).astype(np.uint32)
        lens[g] = len(union)
    return enc, lens


def membership_lists(enc_row, length, G):
    """The per-member row lists that a union entry list encodes."""
    e = np.asarray(enc_row[:length], dtype=np.int64)
    rows = e & ((1 << ROW_BITS) - 1)
    return [rows[((e >> (ROW_BITS + i)) & 1) == 1] for i in range(G)]


def grouped_prefill(q, pool: Pool, enc, lens, G, scale, queries=None):
    """Attention of every prefill query over the rows its membership bit selects from its
    group's union (vLLM PR 63104, "Overview": G = 128 / heads consecutive queries share
    one 128-row tile and gather their union once; "Changes": each query keeps to its own
    top-k through its bit). q: [Q, H, 576] bf16 bits. Returns O [Q', H, 512], LSE [Q', H]
    for `queries` (default: all)."""
    q = np.asarray(q)
    Q = q.shape[0]
    queries = range(Q) if queries is None else queries
    outs, lses = [], []
    for qi in queries:
        g, i = divmod(int(qi), G)
        rows = membership_lists(enc[g], lens[g], G)[i]
        o, l = attention(bf16_bits_to_f64(q[qi]), pool.rows(rows), scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
