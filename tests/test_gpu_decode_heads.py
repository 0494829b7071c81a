"""Decode with 16, 32 and 128 heads on the bf16 MFMA path against the fp64 oracle. A token of up
to 64 heads is one block of 64 head slots, a token of 65 .. 128 heads two blocks, each with its
own splits and merge. Covered: direct output (one split), the merge inside stage 1, stage 2
(more blocks than the workspace's counter words), the fused top-k path, and head slots past H
that must stay unwritten (out and lse are views into buffers whose extra heads hold NaN)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")

BF16_ATOL, RTOL, LSE_ATOL, FP8_ATOL = 2e-2, 1e-2, 1e-3, 6e-2
PAD = 16                                                  # sentinel heads after the real ones


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(seed, H, lens, ns, kv_dtype="bf16", W=2048):
    rng = np.random.default_rng(seed)
    T = len(lens)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32) * 0.5)
    table = np.full((T, W), -1, np.int32)
    for t in range(T):
        table[t, :lens[t]] = rng.choice(ns, size=lens[t], replace=False)
    live = np.unique(table[table >= 0]).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    return q, table, np.asarray(lens, np.int32), live, vals


def _pools(live, vals, ns, kv_dtype):
    kv = smla.KvCache.empty(gc.KV_CODE[kv_dtype], ns)
    src = vals if kv_dtype != "bf16" else wl.f32_to_bf16_bits(vals)
    st, sd = gc.src_tensor(src)
    smla.smla_kv_write(st, _t(live), kv)
    pool = oracle.Pool(ns, kv_dtype)
    oracle.kv_write(pool, src, sd, live)
    return kv, pool


def _padded_outputs(T, H):
    out_full = torch.full((T, H + PAD, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_full = torch.full((T, H + PAD), float("nan"), dtype=torch.float32, device="cuda")
    return out_full, lse_full, out_full[:, :H], lse_full[:, :H]


def _check(out, lse, o_ref, l_ref, atol, what):
    gc.assert_close(out.float().cpu().numpy(), o_ref, atol, RTOL, what + " out")
    gc.assert_lse(lse.cpu().numpy(), l_ref, LSE_ATOL, what + " lse")


@pytest.mark.parametrize("H", [16, 32, 128])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [0, 3])
def test_decode_heads(H, kv_dtype, splits):
    lens = [0, 1, 31, 33, 300, 1025, 1500, 2048]
    ns = 40000
    q, table, lens, live, vals = _case(81 + H, H, lens, ns, kv_dtype)
    kv, pool = _pools(live, vals, ns, kv_dtype)
    T = len(lens)
    out_full, lse_full, out, lse = _padded_outputs(T, H)
    smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16, out=out, lse=lse,
                            num_splits=splits)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    _check(out, lse, o_ref, l_ref, FP8_ATOL if kv_dtype == "fp8" else BF16_ATOL, f"H={H} {kv_dtype} splits={splits}")
    assert bool(torch.all(torch.isnan(out_full[:, H:].float()))) and bool(torch.all(torch.isnan(lse_full[:, H:])))
    assert bool(torch.all(out[0] == 0)) and bool(torch.all(torch.isneginf(lse[0])))   # the empty token


def test_decode_heads_128_topk_fused_equals_two_kernels():
    """The fused top-k decode of 128 heads on the bf16 workload's index lists and page tables is
    bitwise the resolve + decode form; two tokens against the oracle."""
    c = gc.config("decode_bf16_b32")
    lay = c.layout
    kv, _ = gc.gpu_pool(smla, lay, c.rows, "bf16")
    pool, _ = gc.oracle_pool(lay, c.rows, "bf16")
    rng = np.random.default_rng(88)
    q = wl.f32_to_bf16_bits(rng.standard_normal((len(c.idx), 128, 576)).astype(np.float32) * 0.5)
    qt = gc.q_tensor(q, "bf16")
    idx, valid, req, pt, ctx = _t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx)
    slots = smla.smla_resolve_slots(idx, valid, req, pt, ctx, lay.page_size)
    a = smla.smla_sparse_decode(qt, kv, slots, valid, 1, c.scale)
    b = smla.smla_sparse_decode_topk(qt, kv, idx, valid, req, pt, ctx, lay.page_size, c.scale)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oslots = oracle.resolve_slots(c.idx, c.valid, c.tok_req, lay.page_table, lay.ctx, lay.page_size)
    sample = [0, 31]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, oslots[sample], c.valid[sample], 1, c.scale)
    _check(b[0][sample], b[1][sample], o_ref, l_ref, BF16_ATOL, "H=128 fused top-k")


def test_decode_heads_128_stage2():
    """2,049 tokens of 128 heads are 4,098 blocks, more than the workspace's counter words:
    stage 2 merges; a sample of tokens against the oracle, and the pad heads stay unwritten."""
    T, H, ns = 2049, 128, 30000
    rng = np.random.default_rng(89)
    lens = rng.integers(1100, 2049, T)
    q, table, lens, live, vals = _case(89, H, lens, ns)
    kv, pool = _pools(live, vals, ns, "bf16")
    out_full, lse_full, out, lse = _padded_outputs(T, H)
    smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16, out=out, lse=lse,
                            num_splits=2)
    sample = [0, 1, 1024, 2047, 2048]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, table[sample], lens[sample], 1, 1 / 16)
    _check(out[sample], lse[sample], o_ref, l_ref, BF16_ATOL, "H=128 stage 2")
    assert bool(torch.all(torch.isnan(out_full[:, H:].float()))) and bool(torch.all(torch.isnan(lse_full[:, H:])))
