"""Seeded synthetic inputs for sparse MLA over a paged latent KV cache.

This module only draws random numbers and lays them out. It holds none of the
attention, slot-resolution, union or quantisation arithmetic: the CPU oracle and
the HIP path each implement those on their own, and both are fed from here.

Shapes follow the pages' workloads:
  * one latent row per cached token, 512 latent + 64 rotary values (vLLM PR 63104,
    bench_shardq_rank.py: LORA/ROPE constants and the [blocks, 64, 576] cache view);
  * 64 query heads sharing that row, top-k 2048 rows per query (same PR, "Details");
  * a paged cache with 64-slot pages, whose page table is dealt from a seeded
    permutation of the pool, so that logical neighbours are physically scattered.

Every array is numpy; bf16 data is carried as its uint16 bit pattern. Values that
a config stores in bf16 are drawn in float32 and rounded to nearest-even here,
because that is the storage type of the input, not a step of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE
TOPK = 2048
PAGE = 64


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    out = r.astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass
class PagedLayout:
    """Per-request page tables over one pool of `num_slots` slots."""
    page_size: int
    num_slots: int
    page_table: np.ndarray  # int32 [R, max_pages], unused entries -1
    ctx: np.ndarray         # int32 [R] tokens in each request's context


def deal_pages(rng: np.random.Generator, ctx: np.ndarray, page_size: int,
               num_pages: Optional[int] = None, max_pages: Optional[int] = None) -> PagedLayout:
    """Give every request ceil(ctx/page_size) pages taken from a permutation of the pool."""
    need = -(-ctx.astype(np.int64) // page_size)
    total = int(need.sum())
    if num_pages is None:
        num_pages = total
    assert total <= num_pages
    if max_pages is None:
        max_pages = int(need.max())
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.full((len(ctx), max_pages), -1, dtype=np.int32)
    at = 0
    for r, n in enumerate(need):
        pt[r, :n] = perm[at:at + n]
        at += n
    return PagedLayout(page_size, num_pages * page_size, pt, ctx.astype(np.int32))


def sample_unique(rng: np.random.Generator, high: int, k: int) -> np.ndarray:
    """k distinct integers drawn uniformly from [0, high), in random order."""
    return rng.choice(high, size=k, replace=False).astype(np.int32)


def _sample_excluding(rng: np.random.Generator, high: int, k: int, excluded: np.ndarray) -> np.ndarray:
    """k distinct integers drawn uniformly from the values in [0, high) not flagged in
    `excluded`, in draw order (sequential draws, repeats and excluded values rejected)."""
    got = np.zeros(0, np.int64)
    while len(got) < k:
        cand = rng.integers(0, high, size=2 * (k - len(got)) + 64)
        cand = np.concatenate([got, cand[~excluded[cand]]])
        _, first = np.unique(cand, return_index=True)
        got = cand[np.sort(first)]
    return got[:k].astype(np.int32)


@dataclasses.dataclass
class LogicalRows:
    """Cache content in logical form: the row of request `req[i]` at context position
    `pos[i]`. Only positions that some query reads are listed; where the rows land in
    the pool is left to each side's own slot resolution and cache write, and every
    slot that receives no row is poison (NaN)."""
    req: np.ndarray     # int32 [n]
    pos: np.ndarray     # int32 [n]
    values: np.ndarray  # [n, 576]: float32 values, or uint16 bf16 bits


def referenced_positions(req: np.ndarray, idx: np.ndarray, ctx: np.ndarray,
                         dense_reqs=()) -> tuple[np.ndarray, np.ndarray]:
    """Unique (request, position) pairs named by the index lists (entries < 0 skipped),
    plus every position of the requests in `dense_reqs`."""
    r = np.repeat(req.astype(np.int64), idx.shape[1])
    p = idx.reshape(-1).astype(np.int64)
    keep = p >= 0
    keys = [r[keep] * (1 << 32) + p[keep]]
    for d in dense_reqs:
        keys.append(np.int64(d) * (1 << 32) + np.arange(int(ctx[d]), dtype=np.int64))
    k = np.unique(np.concatenate(keys))
    return (k >> 32).astype(np.int32), (k & 0xFFFFFFFF).astype(np.int32)


@dataclasses.dataclass
class DecodeCase:
    name: str
    H: int
    scale: float
    q_dtype: str                 # "f32" | "bf16"
    kv_dtype: str                # "f32" | "bf16" | "fp8"
    q: np.ndarray                # [T, H, 576] float32 or bf16 bits
    layout: PagedLayout
    tok_req: np.ndarray          # int32 [T]
    idx: np.ndarray              # int32 [T, W] logical indices, -1 padded
    valid: np.ndarray            # int32 [T]
    rows: LogicalRows            # cache write source: float32 (f32, fp8 caches) or bf16 bits
    dense_tokens: np.ndarray     # int32 tokens that attend to their whole context (page-table path)


def _normal(rng, shape, scale):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def decode_tiny_f32(seed: int = 1) -> DecodeCase:
    """Tiny fp32 decode: 1 query token, 16 heads, a 4096-slot pool, context 1024,
    256 unique indices, identity page table."""
    rng = np.random.default_rng(seed)
    H, T = 16, 1
    ctx = np.array([1024], np.int32)
    pt = np.full((1, 16), -1, np.int32)
    pt[0, :] = np.arange(16, dtype=np.int32)
    layout = PagedLayout(PAGE, 4096, pt, ctx)
    q = _normal(rng, (T, H, ROW), 1.0)
    idx = sample_unique(rng, 1024, 256)[None, :]
    tok_req = np.zeros(1, np.int32)
    req, pos = referenced_positions(tok_req, idx, ctx)
    rows = LogicalRows(req, pos, _normal(rng, (len(pos), ROW), 1.0))
    return DecodeCase("tiny sparse MLA decode, fp32, 16 heads, top-k 256", H, 1.0 / 16.0, "f32", "f32",
                      q, layout, tok_req, idx.astype(np.int32), np.array([256], np.int32),
                      rows, np.zeros(0, np.int32))


def decode_bf16_b32(seed: int = 2, T: int = 32) -> DecodeCase:
    """bf16 decode: batch 32, 64 heads, contexts U[8K, 32K], 2^20-slot pool in
    64-slot pages dealt from a permutation, 2048 unique causal indices per query."""
    rng = np.random.default_rng(seed)
    H = 64
    ctx = rng.integers(8192, 32768, size=T, endpoint=True).astype(np.int32)
    layout = deal_pages(rng, ctx, PAGE, num_pages=(1 << 20) // PAGE, max_pages=32768 // PAGE)
    idx = np.stack([sample_unique(rng, int(c), TOPK) for c in ctx])
    q = f32_to_bf16_bits(_normal(rng, (T, H, ROW), 0.5))
    tok_req = np.arange(T, dtype=np.int32)
    req, pos = referenced_positions(tok_req, idx, ctx)
    rows = LogicalRows(req, pos, f32_to_bf16_bits(_normal(rng, (len(pos), ROW), 0.5)))
    return DecodeCase(f"sparse MLA decode, bf16, batch {T}, 64 heads, top-k 2048", H, 1.0 / 16.0,
                      "bf16", "bf16", q, layout, tok_req, idx, np.full(T, TOPK, np.int32), rows,
                      np.zeros(0, np.int32))


def decode_ragged_b128(seed: int = 3, T: int = 128) -> DecodeCase:
    """Ragged bf16 decode: batch 128, contexts U[128, 16K], lists of 2048 padded with -1
    (valid = min(ctx, 2048)); 10% of requests attend to their whole context through the
    page table instead."""
    rng = np.random.default_rng(seed)
    H = 64
    ctx = rng.integers(128, 16384, size=T, endpoint=True).astype(np.int32)
    layout = deal_pages(rng, ctx, PAGE)
    n_dense = int(round(0.1 * T))
    dense = np.sort(rng.choice(T, size=n_dense, replace=False)).astype(np.int32)
    idx = np.full((T, TOPK), -1, np.int32)
    valid = np.minimum(ctx, TOPK).astype(np.int32)
    for t in range(T):
        idx[t, :valid[t]] = sample_unique(rng, int(ctx[t]), int(valid[t]))
    q = f32_to_bf16_bits(_normal(rng, (T, H, ROW), 0.5))
    tok_req = np.arange(T, dtype=np.int32)
    sparse_t = np.setdiff1d(np.arange(T), dense)
    req, pos = referenced_positions(tok_req[sparse_t], idx[sparse_t], ctx, dense_reqs=dense)
    rows = LogicalRows(req, pos, f32_to_bf16_bits(_normal(rng, (len(pos), ROW), 0.5)))
    return DecodeCase(f"ragged sparse MLA decode, bf16, batch {T}, 64 heads", H, 1.0 / 16.0, "bf16", "bf16",
                      q, layout, tok_req, idx, valid, rows, dense)


def decode_fp8_b64(seed: int = 5, T: int = 64, ctx_len: int = 65536) -> DecodeCase:
    """fp8-KV decode: batch 64, 64 heads, context 64K each, 2048 unique indices;
    `rows.values` is the float32 cache write source (latent and rope ~ N(0,1))."""
    rng = np.random.default_rng(seed)
    H = 64
    ctx = np.full(T, ctx_len, np.int32)
    layout = deal_pages(rng, ctx, PAGE)
    idx = np.stack([sample_unique(rng, ctx_len, TOPK) for _ in range(T)])
    q = f32_to_bf16_bits(_normal(rng, (T, H, ROW), 1.0))
    tok_req = np.arange(T, dtype=np.int32)
    req, pos = referenced_positions(tok_req, idx, ctx)
    rows = LogicalRows(req, pos, _normal(rng, (len(pos), ROW), 1.0))
    return DecodeCase(f"fp8-KV sparse MLA decode, batch {T}, 64 heads, top-k 2048", H, 1.0 / 16.0,
                      "bf16", "fp8", q, layout, tok_req, idx, np.full(T, TOPK, np.int32), rows,
                      np.zeros(0, np.int32))


@dataclasses.dataclass
class PrefillCase:
    name: str
    H: int
    G: int
    scale: float
    q: np.ndarray           # bf16 bits [Q, H, 576], token-major
    layout: PagedLayout     # one request holding cached + new tokens
    idx: np.ndarray         # int32 [Q, W] logical causal indices
    valid: np.ndarray       # int32 [Q]
    rows: LogicalRows       # bf16 bits, every position of the request


def prefill_grouped_q8192(seed: int = 4, Q: int = 8192, cached: int = 16384, H: int = 64, G: int = 2,
            shared_frac: float = 0.7, W: int = TOPK) -> PrefillCase:
    """Grouped prefill: Q new query tokens at positions cached+i on `cached` cached
    tokens; each query has W causal indices, ~70% shared with its group partners
    (drawn from [0, first member's position]) and the rest its own."""
    rng = np.random.default_rng(seed)
    total = cached + Q
    layout = deal_pages(rng, np.array([total], np.int32), PAGE)
    n_shared = int(round(shared_frac * W))
    idx = np.empty((Q, W), np.int32)
    for g0 in range(0, Q, G):
        first_pos = cached + g0
        shared = sample_unique(rng, first_pos + 1, n_shared)
        taken = np.zeros(total, bool)
        taken[shared] = True
        for q_i in range(g0, min(g0 + G, Q)):
            own = _sample_excluding(rng, cached + q_i + 1, W - n_shared, taken)
            lst = np.concatenate([shared, own])
            rng.shuffle(lst)
            idx[q_i] = lst
    q = f32_to_bf16_bits(_normal(rng, (Q, H, ROW), 0.5))
    pos = np.arange(total, dtype=np.int32)
    rows = LogicalRows(np.zeros(total, np.int32), pos, f32_to_bf16_bits(_normal(rng, (total, ROW), 0.5)))
    return PrefillCase(f"grouped sparse prefill, bf16, {Q} queries on {cached} cached, {H} heads, G={G}",
                       H, G, 1.0 / 16.0, q, layout, idx, np.full(Q, W, np.int32), rows)


def random_slot_lists(seed: int, Q: int, W: int, num_slots: int, overlap: float = 0.5,
                      G: int = 2, pad_frac: float = 0.0) -> tuple[np.ndarray, np.ndarray]:
    """Small physical-slot lists for union tests: consecutive groups share about `overlap`
    of their entries, some lists are shorter than W (tail padded with -1)."""
    rng = np.random.default_rng(seed)
    slots = np.full((Q, W), -1, np.int32)
    valid = np.full(Q, W, np.int32)
    for g0 in range(0, Q, G):
        n_sh = int(overlap * W)
        shared = sample_unique(rng, num_slots, min(n_sh, num_slots))
        for q_i in range(g0, min(g0 + G, Q)):
            n = W if rng.random() >= pad_frac else int(rng.integers(0, W + 1))
            extra = sample_unique(rng, num_slots, min(W, num_slots))
            lst = np.concatenate([shared, extra[~np.isin(extra, shared)]])[:W]
            rng.shuffle(lst)
            slots[q_i, :n] = lst[:n]
            valid[q_i] = n
    return slots, valid
