"""Pins of the CPU oracle: checks against facts fixed outside the oracle itself.

Each check takes the oracle's reference module (or a deliberately broken copy of it)
and raises AssertionError when the module disagrees with the fact. The facts come from
the pages' formulas worked by hand (tests/golden), closed forms of softmax attention,
torch's float64 scaled-dot-product attention on the CPU, brute force with Python sets,
and the fp8 format definition.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _pool_f32(ref, vals):
    pool = ref.Pool(len(vals), ref.KV_F32)
    pool.store(np.arange(len(vals)), {"rows": vals.astype(np.float32)})
    return pool


# ---------------------------------------------------------------- resolve

def check_resolve_golden(ref):
    for line in open(os.path.join(GOLDEN, "resolve_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        P, row, seq, pos, want = [f.strip() for f in line.split("|")]
        row = np.array([int(x) for x in row.split()], np.int32)[None, :]
        got = ref.resolve_slots(np.array([[int(pos)]]), None, np.array([0]), row,
                                np.array([int(seq)]), int(P))
        assert int(got[0, 0]) == int(want), (line, int(got[0, 0]))


def check_resolve_bruteforce(ref, seed=0):
    """Enumerate every (token, entry) of small random tables with explicit Python loops."""
    rng = _rng(seed)
    for P in (1, 2, 4, 64):
        R, T, W, maxp = 3, 5, 9, 4
        pt = rng.integers(-1, 40, size=(R, maxp)).astype(np.int32)
        seq = rng.integers(0, maxp * P + 3, size=R).astype(np.int32)
        req = rng.integers(0, R, size=T).astype(np.int32)
        req[1], req[3] = -1, R                      # tokens whose request is not in the table
        idx = rng.integers(-3, maxp * P + 5, size=(T, W)).astype(np.int32)
        valid = rng.integers(-1, W + 2, size=T).astype(np.int32)
        got = ref.resolve_slots(idx, valid, req, pt, seq, P)
        for t in range(T):
            for j in range(W):
                i, r = int(idx[t, j]), int(req[t])
                want = -1
                if j < valid[t] and 0 <= r < R and 0 <= i < seq[r] and i // P < maxp and pt[r, i // P] >= 0:
                    want = int(pt[r, i // P]) * P + i % P
                assert got[t, j] == want, (P, t, j, got[t, j], want)
        # no `valid` means every entry counts
        got_all = ref.resolve_slots(idx, None, req, pt, seq, P)
        full = ref.resolve_slots(idx, np.full(T, W, np.int32), req, pt, seq, P)
        assert np.array_equal(got_all, full)


def check_identity_table(ref):
    """An identity page table resolves every in-context index to itself."""
    P, ctx = 64, 1024
    pt = np.arange(16, dtype=np.int32)[None, :]
    idx = _rng(3).permutation(ctx)[None, :256].astype(np.int32)
    got = ref.resolve_slots(idx, None, np.array([0]), pt, np.array([ctx]), P)
    assert np.array_equal(got, idx)


# ---------------------------------------------------------------- attention

def _sdpa(q, kv, scale):
    """torch's float64 CPU scaled-dot-product attention: q [H,576] over kv [n,576],
    values = first 512 columns; plus torch.logsumexp of the scaled scores."""
    qt = torch.from_numpy(q)[None, :, None, :]
    k = torch.from_numpy(kv)[None, None].expand(1, q.shape[0], kv.shape[0], kv.shape[1])
    v = torch.from_numpy(np.ascontiguousarray(kv[:, :512]))[None, None].expand(1, q.shape[0], kv.shape[0], 512)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=scale)[0, :, 0, :]
    lse = torch.logsumexp(scale * (torch.from_numpy(q) @ torch.from_numpy(kv).T), dim=1)
    return o.numpy(), lse.numpy()


def check_dense_equals_sdpa(ref, seed=1):
    """A list covering the whole context gives textbook attention over the context."""
    rng = _rng(seed)
    H, ctx, P = 8, 300, 16
    scale = 0.0625
    pages = 32
    vals = rng.standard_normal((pages * P, 576))
    pool = _pool_f32(ref, vals)
    vals32 = vals.astype(np.float32).astype(np.float64)
    pt = rng.permutation(pages).astype(np.int32)[None, :]
    q = rng.standard_normal((1, H, 576)).astype(np.float32)
    ctx_slots = np.array([pt[0, p // P] * P + p % P for p in range(ctx)])
    want_o, want_l = _sdpa(q[0].astype(np.float64), vals32[ctx_slots], scale)
    # dense paged walk
    o, l = ref.sparse_decode(q, "f32", pool, pt, np.array([ctx]), P, scale)
    assert np.allclose(o[0], want_o, atol=1e-12, rtol=0) and np.allclose(l[0], want_l, atol=1e-12, rtol=0)
    # virtual block table: the whole context as a shuffled top-k list of slots
    sl = ref.resolve_slots(rng.permutation(ctx)[None, :].astype(np.int32), None, np.array([0]), pt,
                           np.array([ctx]), P)
    o2, l2 = ref.sparse_decode(q, "f32", pool, sl, np.array([ctx]), 1, scale)
    assert np.allclose(o2[0], want_o, atol=1e-12, rtol=0) and np.allclose(l2[0], want_l, atol=1e-12, rtol=0)


def check_sparse_equals_sdpa(ref, seed=2):
    """A sparse list equals textbook attention over exactly the listed rows."""
    rng = _rng(seed)
    H, n_slots, k = 4, 500, 37
    vals = rng.standard_normal((n_slots, 576))
    pool = _pool_f32(ref, vals)
    q = rng.standard_normal((1, H, 576)).astype(np.float32)
    sl = rng.choice(n_slots, size=k, replace=False).astype(np.int32)
    table = np.full((1, 50), -1, np.int32)
    table[0, :k] = sl
    want_o, want_l = _sdpa(q[0].astype(np.float64), vals.astype(np.float32).astype(np.float64)[sl], 0.1)
    o, l = ref.sparse_decode(q, "f32", pool, table, np.array([50]), 1, 0.1)
    assert np.allclose(o[0], want_o, atol=1e-12, rtol=0) and np.allclose(l[0], want_l, atol=1e-12, rtol=0)


def check_virtual_equals_physical(ref, seed=3):
    """Resolved slots through page size 1 walk the same rows in the same order as the
    page-table walk, so the results are bitwise equal."""
    rng = _rng(seed)
    P, pages, H = 64, 12, 3
    vals = rng.standard_normal((pages * P, 576))
    pool = _pool_f32(ref, vals)
    pt = rng.permutation(pages).astype(np.int32)[None, :]
    for ctx in (1, 63, 64, 65, 700):
        q = rng.standard_normal((1, H, 576)).astype(np.float32)
        sl = ref.resolve_slots(np.arange(ctx, dtype=np.int32)[None, :], None, np.array([0]), pt,
                               np.array([ctx]), P)
        a = ref.sparse_decode(q, "f32", pool, pt, np.array([ctx]), P, 0.07)
        b = ref.sparse_decode(q, "f32", pool, sl, np.array([ctx]), 1, 0.07)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def check_order_invariance(ref, seed=4):
    rng = _rng(seed)
    vals = rng.standard_normal((200, 576))
    pool = _pool_f32(ref, vals)
    q = rng.standard_normal((1, 5, 576)).astype(np.float32)
    sl = rng.choice(200, size=64, replace=False).astype(np.int32)[None, :]
    a = ref.sparse_decode(q, "f32", pool, sl, np.array([64]), 1, 0.2)
    b = ref.sparse_decode(q, "f32", pool, sl[:, rng.permutation(64)], np.array([64]), 1, 0.2)
    assert np.allclose(a[0], b[0], atol=1e-12, rtol=0) and np.allclose(a[1], b[1], atol=1e-12, rtol=0)


def check_split_combine(ref, seed=5):
    """Splitting the rows into S chunks (some empty) and merging by LSE changes nothing."""
    rng = _rng(seed)
    q = rng.standard_normal((6, 576))
    rows = rng.standard_normal((37, 576))
    o1, l1 = ref.attention(q, rows, 0.125)
    for S in (1, 2, 3, 7, 16, 50):
        o, l = ref.split_attention(q, rows, 0.125, S)
        assert np.allclose(o, o1, atol=1e-12, rtol=0) and np.allclose(l, l1, atol=1e-12, rtol=0), S
    # two explicit halves, combined by hand-checked weights
    oa, la = ref.attention(q, rows[:10], 0.125)
    ob, lb = ref.attention(q, rows[10:], 0.125)
    o, l = ref.lse_combine([oa, ob], [la, lb])
    assert np.allclose(l, np.logaddexp(la, lb), atol=1e-12, rtol=0)
    assert np.allclose(o, o1, atol=1e-12, rtol=0)
    # empty parts contribute nothing; all-empty gives O = 0, LSE = -inf
    oe, le = ref.attention(q, rows[:0], 0.125)
    o, l = ref.lse_combine([oe, oa, oe], [le, la, le])
    assert np.allclose(o, oa, atol=1e-12, rtol=0) and np.allclose(l, la, atol=1e-12, rtol=0)
    o, l = ref.lse_combine([oe, oe], [le, le])
    assert np.all(o == 0) and np.all(np.isneginf(l))


def check_softmax_weights(ref, seed=6):
    """Weights exp(s - LSE) are positive and sum to 1, and O is their weighted sum."""
    rng = _rng(seed)
    q = rng.standard_normal((4, 576))
    rows = rng.standard_normal((50, 576))
    o, l = ref.attention(q, rows, 0.05)
    s = 0.05 * q @ rows.T
    p = np.exp(s - l[:, None])
    assert np.allclose(p.sum(1), 1.0, atol=1e-12, rtol=0)
    assert np.allclose(p @ rows[:, :512], o, atol=1e-12, rtol=0)


def check_closed_forms(ref, seed=7):
    rng = _rng(seed)
    rows = rng.standard_normal((20, 576))
    # q = 0: uniform weights -> mean of the values, LSE = ln n
    o, l = ref.attention(np.zeros((2, 576)), rows, 0.3)
    assert np.allclose(o, rows[:, :512].mean(0)[None], atol=1e-12, rtol=0)
    assert np.allclose(l, math.log(20), atol=1e-12, rtol=0)
    # identical keys: O = the value, LSE = tau q.k + ln n
    q = rng.standard_normal((3, 576))
    same = np.repeat(rows[:1], 7, axis=0)
    o, l = ref.attention(q, same, 0.3)
    assert np.allclose(o, np.repeat(rows[:1, :512], 3, axis=0), atol=1e-12, rtol=0)
    assert np.allclose(l, 0.3 * q @ rows[0] + math.log(7), atol=1e-12, rtol=0)
    # one row: O = its value, LSE = its score
    o, l = ref.attention(q, rows[3:4], 0.3)
    assert np.allclose(o, np.repeat(rows[3:4, :512], 3, axis=0), atol=1e-12, rtol=0)
    assert np.allclose(l, 0.3 * q @ rows[3], atol=1e-12, rtol=0)
    # two rows, scores 2 and 3 only through latent column 0 and rope column 512
    q = np.zeros((1, 576)); q[0, 0] = 2.0; q[0, 512] = 1.0
    r = np.zeros((2, 576)); r[0, 0] = 1.0; r[1, 512] = 3.0; r[0, 5] = 10.0; r[1, 6] = -4.0
    o, l = ref.attention(q, r, 1.0)
    w0 = 1.0 / (1.0 + math.exp(1.0))
    assert abs(l[0] - (3.0 + math.log1p(math.exp(-1.0)))) < 1e-12
    assert abs(o[0, 5] - 10.0 * w0) < 1e-12 and abs(o[0, 6] + 4.0 * (1 - w0)) < 1e-12
    assert abs(o[0, 0] - w0) < 1e-12 and np.count_nonzero(o) == 3
    # no rows: O = 0, LSE = -inf
    o, l = ref.attention(q, r[:0], 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def check_padding_masks(ref, seed=8):
    """Entries past `lens` and negative entries are never read (their rows are poison)."""
    rng = _rng(seed)
    vals = rng.standard_normal((64, 576))
    pool = ref.Pool(128, ref.KV_F32)
    pool.store(np.arange(64), {"rows": vals.astype(np.float32)})   # slots 64.. are NaN
    q = rng.standard_normal((1, 2, 576)).astype(np.float32)
    table = np.array([[3, -1, 7, 100, 120]], np.int32)
    o, l = ref.sparse_decode(q, "f32", pool, table, np.array([3]), 1, 0.1)
    want = ref.attention(q[0].astype(np.float64), vals.astype(np.float32).astype(np.float64)[[3, 7]], 0.1)
    assert np.allclose(o[0], want[0], atol=1e-12, rtol=0) and np.allclose(l[0], want[1], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- union

def _parse_union_line(line):
    G, ns, members, expect = [f.strip() for f in line.split("|")]
    lists = []
    for m in members.split(";"):
        v, lst = m.split(":")
        lists.append((int(v), [int(x) for x in lst.split()]))
    n, ents = expect.split(":")
    return int(G), int(ns), lists, int(n), [int(x, 16) for x in ents.split()]


def check_union_golden(ref):
    for line in open(os.path.join(GOLDEN, "union_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        G, ns, lists, n, ents = _parse_union_line(line)
        W = max(len(l) for _, l in lists)
        slots = np.full((len(lists), W), -1, np.int64)
        for i, (_, l) in enumerate(lists):
            slots[i, :len(l)] = l
        valid = np.array([v for v, _ in lists])
        enc, lens = ref.group_union(slots, valid, G, ns)
        assert lens.shape == (1,) and lens[0] == n, line
        assert [int(e) for e in enc[0, :n]] == ents, (line, [hex(int(e)) for e in enc[0, :n]])


def check_union_bruteforce(ref, seed=9):
    """Python sets, entry by entry, on random small groups (G = 1, 2, 4, 8; tails)."""
    rng = _rng(seed)
    for G in (1, 2, 4, 8):
        Q, W, ns = 2 * G + 1, 12, 40
        slots = rng.integers(-2, ns + 3, size=(Q, W))
        valid = rng.integers(-1, W + 2, size=Q)
        enc, lens = ref.group_union(slots, valid, G, ns)
        assert enc.shape == (-(-Q // G), G * W)
        for g in range(-(-Q // G)):
            sets = []
            for i in range(G):
                qi = g * G + i
                s = set()
                if qi < Q:
                    for j in range(W):
                        if j < valid[qi] and 0 <= slots[qi, j] < ns:
                            s.add(int(slots[qi, j]))
                sets.append(s)
            u = sorted(set().union(*sets))
            assert lens[g] == len(u)
            for k, r in enumerate(u):
                mask = sum(1 << i for i in range(G) if r in sets[i])
                assert int(enc[g, k]) == r + (mask << 24), (G, g, k)


def check_union_special(ref, seed=10):
    rng = _rng(seed)
    lst = rng.choice(1000, size=30, replace=False)
    # G = 1: the list sorted, bit 0 set
    enc, lens = ref.group_union(lst[None, :], np.array([30]), 1, 1000)
    assert lens[0] == 30 and np.array_equal(enc[0, :30], np.sort(lst) + (1 << 24))
    # identical lists: n entries, all bits set
    enc, lens = ref.group_union(np.stack([lst] * 4), np.full(4, 30), 4, 1000)
    assert lens[0] == 30 and np.array_equal(enc[0, :30], np.sort(lst) + (0xF << 24))
    # disjoint lists: sizes add up
    a, b = lst[:15], lst[15:]
    enc, lens = ref.group_union(np.stack([a, b]), np.full(2, 15), 2, 1000)
    assert lens[0] == 30


# ---------------------------------------------------------------- grouped prefill

def check_grouped_equals_decode(ref, seed=11):
    """Each query of a group, masked by its bit, equals decode over its own list."""
    rng = _rng(seed)
    H, W, ns, G = 4, 20, 120, 2
    vals = rng.standard_normal((ns, 576))
    pool = ref.Pool(ns, ref.KV_BF16)
    pool.store(np.arange(ns), {"rows": ref.f32_to_bf16_rne(vals.astype(np.float32))})
    for Q in (4, 5):
        slots = np.full((Q, W), -1, np.int32)
        valid = rng.integers(0, W + 1, size=Q).astype(np.int32)
        for qi in range(Q):
            slots[qi, :valid[qi]] = rng.choice(ns, size=valid[qi], replace=False)
        q = ref.f32_to_bf16_rne(rng.standard_normal((Q, H, 576)).astype(np.float32))
        enc, lens = ref.group_union(slots, valid, G, ns)
        o, l = ref.grouped_prefill(q, pool, enc, lens, G, 0.1)
        od, ld = ref.sparse_decode(q, "bf16", pool, slots, valid, 1, 0.1)
        assert np.allclose(o, od, atol=1e-12, rtol=0)
        assert np.allclose(l, ld, atol=1e-12, rtol=0, equal_nan=False) or \
            np.array_equal(np.isneginf(l), np.isneginf(ld))


# ---------------------------------------------------------------- formats and cache write

def check_e4m3_golden(ref):
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        got = ref.e4m3_decode(np.array([int(c, 16)], np.uint8))[0]
        want = float(v)
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got)
            assert int(ref.e4m3_encode(np.array([want]))[0]) == int(c, 16), c


def check_e4m3_vs_torch(ref):
    """All 256 codes decode as torch's float8_e4m3fn does; encoding matches torch's
    round-to-nearest-even cast wherever that cast does not overflow to NaN."""
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = ref.e4m3_decode(codes)
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    fin = ~np.isnan(tv)
    assert np.array_equal(tv[fin], ov[fin])
    x = np.concatenate([_rng(12).standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    # every midpoint between consecutive finite values, to exercise ties
    pos = np.sort(np.unique(np.abs(ov[fin])))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids, pos, -pos]).astype(np.float32)
    x = x[np.abs(x) <= 464]      # torch's cast turns larger values into NaN
    tc = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    oc = ref.e4m3_encode(x)
    assert np.array_equal(tc, oc), np.flatnonzero(tc != oc)[:5]
    # round trip and saturation
    finite_codes = codes[fin]
    assert np.array_equal(ref.e4m3_encode(ref.e4m3_decode(finite_codes)), finite_codes)
    assert ref.e4m3_encode(np.array([1e6]))[0] == 0x7E and ref.e4m3_encode(np.array([-500.0]))[0] == 0xFE


def check_bf16_vs_torch(ref):
    x = np.concatenate([_rng(13).standard_normal(200000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, 2.0 ** -130], np.float32)])
    # exact ties: low 16 bits = 0x8000 with both parities of the kept part
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000 | 0x3F800000).view(np.float32)
    x = np.concatenate([x, ties])
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ob = ref.f32_to_bf16_rne(x)
    assert np.array_equal(tb, ob)
    assert np.array_equal(ref.bf16_bits_to_f64(ob), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def check_kv_write_fp8(ref, seed=14):
    rng = _rng(seed)
    src = rng.standard_normal((50, 576)).astype(np.float32)
    src[7, :512] = 0.0                       # all-zero latent: scale 0, codes 0
    src[9, 100] = -5.0 * np.abs(src[9, :512]).max()   # negative amax element
    pool = ref.Pool(100, ref.KV_FP8)
    sm = rng.choice(100, size=50, replace=False)
    sm[3] = -1                               # skipped row
    ref.kv_write(pool, src, ref.KV_F32, sm)
    live = np.flatnonzero(sm >= 0)
    st = pool.stored(sm[live])
    amax = np.abs(src[live, :512]).max(1)
    assert np.array_equal(st["scale"], (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    dec = ref.e4m3_decode(st["lat8"])
    for k, i in enumerate(live):
        if amax[k] == 0:
            assert np.all(st["lat8"][k] == 0)
            continue
        j = int(np.argmax(np.abs(src[i, :512])))
        assert abs(dec[k, j]) == 448.0                 # the amax element lands on +-448
        assert np.all(np.abs(dec[k]) <= 448.0)
        # each code is the nearest e4m3 value to the float32 quotient
        quot = (src[i, :512] / st["scale"][k]).astype(np.float64)
        assert np.all(np.abs(dec[k] - quot) <= np.abs(quot) * 2.0 ** -4 + 2.0 ** -10)
    assert np.array_equal(st["rope16"], ref.f32_to_bf16_rne(src[live, 512:]))
    # dequantised rows are within half an e4m3 step of the source
    rows = pool.rows(sm[live])
    err = np.abs(rows[:, :512] - src[live, :512])
    assert np.all(err <= np.abs(src[live, :512]) * 2.0 ** -4 + amax[:, None] / 448 * 2.0 ** -10)
    # the skipped row (slot -1) wrote nothing: every slot outside the written ones still reads NaN
    unwritten = np.setdiff1d(np.arange(100), sm[live])
    assert len(unwritten) == 51 and np.all(np.isnan(pool.rows(unwritten)))


def check_kv_write_bf16(ref, seed=15):
    rng = _rng(seed)
    src = rng.standard_normal((10, 576)).astype(np.float32)
    pool = ref.Pool(20, ref.KV_BF16)
    ref.kv_write(pool, src, ref.KV_F32, np.arange(10) * 2)
    st = pool.stored(np.arange(10) * 2)
    tb = torch.from_numpy(src).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(st["rows"], tb)
    assert np.all(np.isnan(pool.rows(np.array([1, 3]))))


ALL_CHECKS = [v for k, v in dict(globals()).items() if k.startswith("check_")]
