"""Slot resolution and group unions on the GPU, bit-exact against the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import oracle_pins
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_resolve_golden():
    for line in open(os.path.join(GOLDEN, "resolve_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        P, row, seq, pos, want = [f.strip() for f in line.split("|")]
        pt = np.array([[int(x) for x in row.split()]], np.int32)
        got = smla.smla_resolve_slots(_t(np.array([[int(pos)]], np.int32)), None, _t(np.zeros(1, np.int32)),
                                      _t(pt), _t(np.array([int(seq)], np.int32)), int(P))
        assert int(got.cpu()[0, 0]) == int(want), line


@pytest.mark.parametrize("P", [1, 2, 16, 64])
def test_resolve_random(P):
    rng = np.random.default_rng(100 + P)
    R, T, W, maxp = 7, 33, 300, 9
    pt = rng.integers(-1, 500, size=(R, maxp)).astype(np.int32)
    seq = rng.integers(0, maxp * P + 3, size=R).astype(np.int32)
    req = rng.integers(-1, R + 1, size=T).astype(np.int32)          # includes out-of-range requests
    idx = rng.integers(-3, maxp * P + 5, size=(T, W)).astype(np.int32)
    valid = rng.integers(-1, W + 2, size=T).astype(np.int32)
    got = smla.smla_resolve_slots(_t(idx), _t(valid), _t(req), _t(pt), _t(seq), P).cpu().numpy()
    # tokens whose request id is not a row of the page table resolve to all -1 on both sides
    okreq = (req >= 0) & (req < R)
    want = oracle.resolve_slots(idx, valid, req, pt, seq, P)
    assert np.all(want[~okreq] == -1)
    assert np.array_equal(got, want)
    got2 = smla.smla_resolve_slots(_t(idx), None, _t(np.where(okreq, req, 0).astype(np.int32)), _t(pt), _t(seq), P)
    assert np.array_equal(got2.cpu().numpy(), oracle.resolve_slots(idx, None, np.where(okreq, req, 0), pt, seq, P))


def test_resolve_strided_rows():
    rng = np.random.default_rng(7)
    base = rng.integers(0, 1000, size=(6, 50)).astype(np.int32)
    idx = _t(base)[:, 5:45]                       # row stride 50, width 40
    pt = np.arange(1000, dtype=np.int32)[None, :]
    out = torch.full((6, 64), 12345, dtype=torch.int32, device="cuda")
    smla.smla_resolve_slots(idx, None, _t(np.zeros(6, np.int32)), _t(pt), _t(np.array([1000], np.int32)), 1,
                            slots=out[:, 8:48])
    o = out.cpu().numpy()
    assert np.array_equal(o[:, 8:48], base[:, 5:45])
    assert np.all(o[:, :8] == 12345) and np.all(o[:, 48:] == 12345)


@pytest.mark.parametrize("cfg", ["decode_bf16_b32", "prefill_grouped_q8192"])
def test_resolve_config(cfg):
    if cfg == "decode_bf16_b32":
        c = gc.config("decode_bf16_b32")
        idx, req, valid = c.idx, c.tok_req, c.valid
    else:
        c = wl.prefill_grouped_q8192(Q=2048, cached=16384)
        idx, req, valid = c.idx, np.zeros(c.idx.shape[0], np.int32), c.valid
    lay = c.layout
    got = smla.smla_resolve_slots(_t(idx), _t(valid), _t(req), _t(lay.page_table), _t(lay.ctx), lay.page_size)
    want = oracle.resolve_slots(idx, valid, req, lay.page_table, lay.ctx, lay.page_size)
    assert np.array_equal(got.cpu().numpy(), want)


def _union_gpu(slots, valid, G, num_slots):
    enc, lens = smla.smla_build_group_union(_t(slots.astype(np.int32)), None if valid is None else _t(valid.astype(np.int32)),
                                            G, num_slots)
    return enc.cpu().numpy().view(np.uint32), lens.cpu().numpy()


def _compare_union(enc_g, lens_g, enc_o, lens_o):
    assert np.array_equal(lens_g, lens_o)
    for g in range(len(lens_o)):
        n = lens_o[g]
        assert np.array_equal(enc_g[g, :n], enc_o[g, :n]), g


def test_union_golden():
    for line in open(os.path.join(GOLDEN, "union_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        G, ns, lists, n, ents = oracle_pins._parse_union_line(line)
        if G not in (2, 4, 8):
            continue
        W = max(len(l) for _, l in lists)
        slots = np.full((len(lists), W), -1, np.int32)
        for i, (_, l) in enumerate(lists):
            slots[i, :len(l)] = l
        valid = np.array([v for v, _ in lists], np.int32)
        enc, lens = _union_gpu(slots, valid, G, ns)
        assert lens[0] == n, line
        assert [int(e) for e in enc[0, :n]] == ents, line


@pytest.mark.parametrize("G,ns", [(2, 5000), (8, 5000), (8, 262143), (4, 1 << 20)])
def test_union_strided_lists(G, ns):
    """Lists read from a column slice of a wider table (row stride W + 37), both builders."""
    rng = np.random.default_rng(G * 131 + ns % 977)
    Q, W = 13, 2048 if G != 4 else 1024
    wide = np.full((Q, W + 37), 77, np.int32)
    for q in range(Q):
        wide[q, :W] = rng.choice(ns, size=W, replace=False)
    wide[3, 100:200] = -1
    valid = rng.integers(0, W + 1, size=Q).astype(np.int32)
    t = _t(wide)[:, :W]
    assert t.stride(0) == W + 37
    enc, lens = smla.smla_build_group_union(t, _t(valid), G, ns)
    enc_o, lens_o = oracle.group_union(wide[:, :W], valid, G, ns)
    _compare_union(enc.cpu().numpy().view(np.uint32), lens.cpu().numpy(), enc_o, lens_o)


@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("Q", [1, 7, 64])
@pytest.mark.parametrize("ns", [5000, 262143, 262144, 1 << 20, (1 << 20) + 1, 3000000])
def test_union_random(G, Q, ns):
    # pools of up to 2^20 rows take the bit-map kernel (with 16,384 entries per group, G = 8 here,
    # in windows of 2^18 rows), larger ones the sorting kernel
    W = 1024 if G == 4 else 2048
    slots, valid = wl.random_slot_lists(1000 + G * 10 + Q, Q, W, ns, overlap=0.6, G=G, pad_frac=0.3)
    rng = np.random.default_rng(Q)
    # sprinkle negative rows, rows past the pool and in-list duplicates; every list holds the
    # pool's last row
    m = rng.random(slots.shape)
    slots[m < 0.01] = -5
    slots[(m > 0.01) & (m < 0.02)] = ns + 3
    slots[:, 1] = slots[:, 0]
    slots[:, 2] = ns - 1
    enc_g, lens_g = _union_gpu(slots, valid, G, ns)
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    _compare_union(enc_g, lens_g, enc_o, lens_o)
    enc_g2, lens_g2 = _union_gpu(slots, None, G, ns)
    enc_o2, lens_o2 = oracle.group_union(slots, np.full(Q, W), G, ns)
    _compare_union(enc_g2, lens_g2, enc_o2, lens_o2)


@pytest.mark.parametrize("ns", [262145, 600000, 1 << 20])
def test_union_windows(ns):
    """Groups of 8 lists of 2,048 entries map the pool in windows of 2^18 rows: rows on both
    sides of every window edge, the pool's first and last rows and a short last window, each
    listed by some members only, against the oracle."""
    rng = np.random.default_rng(ns % 1009)
    Q, W, G = 16, 2048, 8
    edges = [r for k in range(1, 4) for r in ((k << 18) - 1, k << 18) if r < ns] + [0, ns - 1]
    slots = np.stack([rng.choice(ns, size=W, replace=False) for _ in range(Q)]).astype(np.int32)
    for q in range(Q):
        pick = [e for i, e in enumerate(edges) if (q + i) % 3 != 0]          # some members only
        row = slots[q][~np.isin(slots[q], edges)][: W - len(pick)]
        slots[q] = np.concatenate([np.array(pick, np.int32), row])
        rng.shuffle(slots[q])
    valid = np.full(Q, W, np.int32)
    valid[5] = 1000
    enc_g, lens_g = _union_gpu(slots, valid, G, ns)
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    _compare_union(enc_g, lens_g, enc_o, lens_o)


def test_union_24bit_rows():
    ns = (1 << 24) - 2
    rng = np.random.default_rng(5)
    slots = rng.integers(ns - 3000, ns, size=(6, 512)).astype(np.int32)
    slots[0, :3] = [ns - 1, ns, 0]
    enc_g, lens_g = _union_gpu(slots, None, 2, ns)
    enc_o, lens_o = oracle.group_union(slots, np.full(6, 512), 2, ns)
    _compare_union(enc_g, lens_g, enc_o, lens_o)


def test_union_prefill_grouped_q8192():
    c = gc.config("prefill_grouped_q8192")
    lay = c.layout
    sl = oracle.resolve_slots(c.idx, c.valid, np.zeros(len(c.idx), np.int32), lay.page_table, lay.ctx, lay.page_size)
    enc_g, lens_g = _union_gpu(sl, c.valid, 2, lay.num_slots)
    enc_o, lens_o = oracle.group_union(sl, c.valid, 2, lay.num_slots)
    _compare_union(enc_g, lens_g, enc_o, lens_o)
    assert 1.2 < lens_o.mean() / 2048 < 1.35
