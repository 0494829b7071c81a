"""Seeded random shapes through the decode entry points against the fp64 oracle. Each case draws
its own batch, head count (16, 32, 64, 128), cache format (bf16, or fp8 packed or in separate
planes), page size (1, 16, 64), table width, per-token lengths (zero, full and anything
between), table holes and out-of-range entries, split count (chosen or forced), and softmax
scale. Every case runs the decode over its table, and a case that has a page table also runs
the fused top-k form, which must equal resolve + decode bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")

BF16_ATOL, RTOL, LSE_ATOL, FP8_ATOL = 2e-2, 1e-2, 1e-3, 6e-2
N_CASES = 24


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class PlanarKv:
    """An fp8 pool as three separate planes with padded strides (the descriptor's general form)."""

    def __init__(self, packed):
        n = packed.num_slots
        self.dtype, self.num_slots = smla.SMLA_FP8_E4M3, n
        self.lat = torch.full((n, 528), 0x7F, dtype=torch.uint8, device="cuda")
        self.rope = torch.full((n, 80), 0x7FC0, dtype=torch.int16, device="cuda")
        self.sc = torch.full((n, 3), float("nan"), dtype=torch.float32, device="cuda")
        self.lat[:, :512].copy_(packed.lat8())
        self.rope[:, :64].copy_(packed.rope16())
        self.sc[:, 0].copy_(packed.scale())

    def desc(self):
        d = smla.smla.smla_kv()
        d.dtype, d.num_slots = self.dtype, self.num_slots
        d.lat8, d.lat8_stride = self.lat.data_ptr(), 528
        d.rope16, d.rope16_stride = self.rope.data_ptr(), 160
        d.scale, d.scale_stride = self.sc.data_ptr(), 12
        return d


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.choice([1, 2, 3, 5, 8, 13, 32]))
    H = int(rng.choice([16, 32, 64, 128]))
    kv_dtype = str(rng.choice(["bf16", "fp8", "fp8-planes"]))
    P = int(rng.choice([1, 16, 64]))
    splits = int(rng.choice([0, 0, 1, 2, 5, 16]))
    scale = float(rng.choice([1 / 16, 1 / 24, 0.1]))
    return rng, T, H, kv_dtype, P, splits, scale


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_decode_shape(seed):
    rng, T, H, kv_dtype, P, splits, scale = _case(seed)
    fmt = "fp8" if kv_dtype.startswith("fp8") else "bf16"
    R = T                                                   # one request per token
    max_ctx = int(rng.choice([64, 700, 2048, 3000]))
    ptw = -(-max_ctx // P)                                 # page-table width (pages per request)
    num_pages = R * ptw + 8
    num_slots = num_pages * P
    ctx = rng.integers(0, max_ctx + 1, size=R).astype(np.int32)
    ctx[rng.integers(0, R)] = max_ctx                      # one full-length request
    if R > 2:
        ctx[rng.integers(0, R)] = 0                        # and an empty one
    page_table = rng.permutation(num_pages)[:R * ptw].reshape(R, ptw).astype(np.int32)
    if R > 1:
        page_table[rng.integers(0, R), rng.integers(0, ptw)] = -1       # a hole in the table
    # top-k lists over each request's context (width W >= the largest valid count), with
    # padding, negative and past-the-context entries inside the valid prefix
    W = int(min(2048, max(1, max_ctx)))
    valid = np.minimum(ctx, W).astype(np.int32)
    idx = np.full((T, W), -1, np.int32)
    for t in range(T):
        v = int(valid[t])
        if v:
            idx[t, :v] = rng.choice(max(int(ctx[t]), 1), size=v, replace=False)
            if v > 3:
                idx[t, rng.integers(0, v)] = -3
                idx[t, rng.integers(0, v)] = int(ctx[t]) + 5
    tok_req = np.arange(T, dtype=np.int32)
    # rows for every slot a page table names
    live = np.unique((page_table[page_table >= 0][:, None] * P + np.arange(P)[None, :]).reshape(-1)).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * (1.0 if fmt == "fp8" else 0.5)
    kv = smla.KvCache.empty(gc.KV_CODE[fmt], num_slots)
    src = vals if fmt == "fp8" else wl.f32_to_bf16_bits(vals)
    st, sd = gc.src_tensor(src)
    smla.smla_kv_write(st, _t(live), kv)
    pool = oracle.Pool(num_slots, fmt)
    oracle.kv_write(pool, src, sd, live)
    if kv_dtype == "fp8-planes":
        kv = PlanarKv(kv)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32) * 0.5)
    qt = gc.q_tensor(q, "bf16")
    atol = FP8_ATOL if fmt == "fp8" else BF16_ATOL
    what = f"seed {seed}: T={T} H={H} {kv_dtype} P={P} splits={splits} max_ctx={max_ctx}"
    # dense paged decode: the page-table rows, length = context
    out, lse = smla.smla_sparse_decode(qt, kv, _t(page_table), _t(ctx), P, scale,
                                       num_splits=min(splits, -(-ptw * P // 32)))
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, page_table, ctx, P, scale)
    gc.assert_close(out.float().cpu().numpy(), o_ref, atol, RTOL, what + " dense out")
    gc.assert_lse(lse.cpu().numpy(), l_ref, LSE_ATOL, what + " dense lse")
    # sparse top-k: resolve + decode, and the fused form
    args = (_t(idx), _t(valid), _t(tok_req), _t(page_table), _t(ctx))
    slots = smla.smla_resolve_slots(*args, P)
    oslots = oracle.resolve_slots(idx, valid, tok_req, page_table, ctx, P)
    assert np.array_equal(slots.cpu().numpy(), oslots), what
    sp = min(splits, -(-W // 32))
    a = smla.smla_sparse_decode(qt, kv, slots, _t(valid), 1, scale, num_splits=sp)
    b = smla.smla_sparse_decode_topk(qt, kv, *args, P, scale, num_splits=sp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), what
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, oslots, valid, 1, scale)
    gc.assert_close(b[0].float().cpu().numpy(), o_ref, atol, RTOL, what + " top-k out")
    gc.assert_lse(b[1].cpu().numpy(), l_ref, LSE_ATOL, what + " top-k lse")


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_shape(seed):
    """Union build + grouped prefill on random shapes: G in {2, 4, 8} (H = 128 / G), a query
    count that may leave the last group short, list widths, empty and partial lists, list
    overlap, pools of several sizes (the bit-map union builder; the sorting one is covered by the
    union tests), and every cache format."""
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([2, 4, 8]))
    H = 128 // G
    Q = int(rng.integers(1, 4 * G + 1))
    W = int(rng.choice([32, 300, 1024, 2048]))
    ns = int(rng.choice([3000, 40000, 200000]))
    kv_dtype = str(rng.choice(["bf16", "fp8", "fp8-planes"]))
    fmt = "fp8" if kv_dtype.startswith("fp8") else "bf16"
    overlap = float(rng.choice([0.0, 0.5, 0.9]))
    slots, valid = wl.random_slot_lists(3000 + seed, Q, W, ns, overlap=overlap, G=G, pad_frac=0.3)
    if Q > 1:
        valid[rng.integers(0, Q)] = 0
    live = np.unique(slots[slots >= 0]).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * (1.0 if fmt == "fp8" else 0.5)
    kv = smla.KvCache.empty(gc.KV_CODE[fmt], ns)
    src = vals if fmt == "fp8" else wl.f32_to_bf16_bits(vals)
    st, sd = gc.src_tensor(src)
    smla.smla_kv_write(st, _t(live), kv)
    pool = oracle.Pool(ns, fmt)
    oracle.kv_write(pool, src, sd, live)
    if kv_dtype == "fp8-planes":
        kv = PlanarKv(kv)
    q = wl.f32_to_bf16_bits(rng.standard_normal((Q, H, 576)).astype(np.float32) * 0.5)
    scale = float(rng.choice([1 / 16, 0.1]))
    what = f"seed {seed}: G={G} Q={Q} W={W} ns={ns} {kv_dtype} overlap={overlap}"
    enc, lens = smla.smla_build_group_union(_t(slots), _t(valid), G, ns)
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    lens_g = lens.cpu().numpy()
    assert np.array_equal(lens_g, lens_o), what
    enc_g = enc.cpu().numpy().view(np.uint32)
    for g in range(len(lens_o)):
        assert np.array_equal(enc_g[g, :lens_o[g]], enc_o[g, :lens_o[g]].view(np.uint32)), what + f" group {g}"
    out, lse = smla.smla_grouped_prefill(gc.q_tensor(q, "bf16"), kv, enc, lens, G, scale)
    o_ref, l_ref = oracle.grouped_prefill(q, pool, enc_o, lens_o, G, scale)
    atol = FP8_ATOL if fmt == "fp8" else BF16_ATOL
    gc.assert_close(out.float().cpu().numpy(), o_ref, atol, RTOL, what + " out")
    gc.assert_lse(lse.cpu().numpy(), l_ref, LSE_ATOL, what + " lse")
