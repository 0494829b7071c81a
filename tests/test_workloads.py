"""The seeded generators produce the shapes and structure the configs describe (CPU)."""
import numpy as np

import workloads as wl
import oracle


def test_decode_tiny_f32_shapes():
    c = wl.decode_tiny_f32()
    assert c.q.shape == (1, 16, 576) and c.q.dtype == np.float32
    assert c.idx.shape == (1, 256) and len(np.unique(c.idx)) == 256
    assert c.idx.min() >= 0 and c.idx.max() < 1024
    assert c.rows.values.shape == (256, 576)


def test_decode_bf16_b32_structure():
    c = wl.decode_bf16_b32()
    assert c.q.shape == (32, 64, 576) and c.q.dtype == np.uint16
    assert np.all((c.layout.ctx >= 8192) & (c.layout.ctx <= 32768))
    assert c.layout.num_slots == 1 << 20
    for t in range(32):
        row = c.idx[t]
        assert len(np.unique(row)) == 2048 and row.min() >= 0 and row.max() < c.layout.ctx[t]
    used = c.layout.page_table[c.layout.page_table >= 0]
    assert len(np.unique(used)) == len(used)          # no page is dealt twice
    assert len(c.rows.pos) == 32 * 2048


def test_decode_ragged_b128_structure():
    c = wl.decode_ragged_b128(T=24)
    assert np.array_equal(c.valid, np.minimum(c.layout.ctx, 2048))
    for t in range(24):
        v = c.valid[t]
        assert np.all(c.idx[t, v:] == -1)
        assert len(np.unique(c.idx[t, :v])) == v and c.idx[t, :v].max() < c.layout.ctx[t]
    assert len(c.dense_tokens) == round(0.1 * 24)


def test_prefill_grouped_q8192_overlap():
    c = wl.prefill_grouped_q8192(Q=256, cached=4096)
    assert c.idx.shape == (256, 2048)
    for qi in range(256):
        assert len(np.unique(c.idx[qi])) == 2048
        assert c.idx[qi].max() <= 4096 + qi                 # causal, own position included
    enc, lens = oracle.group_union(c.idx, c.valid, 2, 1 << 24)
    ratio = lens.mean() / 2048
    assert 1.2 < ratio < 1.3     # 1434 shared + 2 * 614 own, less own picks that collide


def test_decode_fp8_b64_structure():
    c = wl.decode_fp8_b64(T=4, ctx_len=65536)
    assert c.kv_dtype == "fp8" and c.rows.values.dtype == np.float32
    assert c.layout.num_slots == 4 * 65536


def test_seeded():
    a, b = wl.decode_bf16_b32(T=4), wl.decode_bf16_b32(T=4)
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.q, b.q)
