"""Pools on both sides of 2^32 bytes. Stage 1 reads a pool of at most 2^32 bytes by row index
through a buffer resource (its hardware offset is 32 bits wide) and a larger one through
per-lane 64-bit addresses; both must gather the same rows. The slot lists hold the pool's last
row, the rows on both sides of the first row whose byte offset passes 2^32 (which a 32-bit
offset would wrap onto row 0's neighbourhood), -1 holes and random rows. Unused slots hold
NaN, so a wrong gather cannot pass. Tolerances as in the decode tests."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")

BF16_ATOL, BF16_RTOL, LSE_ATOL, FP8_ATOL = 2e-2, 1e-2, 1e-3, 6e-2
ROW_BYTES = {"bf16": 1152, "fp8": 640}        # the default bf16 row and the aligned fp8 row


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _edge_slots(num_slots, kv_dtype):
    wrap = -(-(1 << 32) // ROW_BYTES[kv_dtype])       # first row whose offset passes 2^32
    s = [0, num_slots - 1, num_slots - 2, wrap - 1, wrap, wrap + 1]
    return [x for x in s if 0 <= x < num_slots]


def _lists(rng, T, W, lens, num_slots, kv_dtype):
    table = np.full((T, W), -1, np.int32)
    edge = _edge_slots(num_slots, kv_dtype)
    for t in range(T):
        n = min(int(lens[t]), W)
        rest = rng.choice(num_slots, size=n + len(edge), replace=False)
        rest = rest[~np.isin(rest, edge)][: n - len(edge)]
        row = np.concatenate([np.array(edge, np.int64), rest])
        rng.shuffle(row)
        table[t, :n] = row[:n]
        table[t, rng.integers(0, n)] = -1               # a hole inside the valid prefix
    return table


def _pool(live, vals, num_slots, kv_dtype):
    kv = smla.KvCache.empty(gc.KV_CODE[kv_dtype], num_slots)
    src = vals if kv_dtype != "bf16" else wl.f32_to_bf16_bits(vals)
    st, sd = gc.src_tensor(src)
    smla.smla_kv_write(st, _t(live), kv)
    pool = oracle.Pool(num_slots, kv_dtype)
    oracle.kv_write(pool, src, sd, live)
    return kv, pool


@pytest.mark.parametrize("kv_dtype,num_slots", [
    ("bf16", (1 << 32) // 1152),          # 2^32 - 768 bytes: read by index, up to the last row
    ("bf16", 4_000_000),                  # 4.6 GB: 64-bit addresses
    ("fp8", (1 << 32) // 640),            # 2^32 - 256 bytes of aligned fp8 rows
    ("fp8", 7_000_000),                   # 4.5 GB
])
def test_decode_pool_at_4gib(kv_dtype, num_slots):
    rng = np.random.default_rng(num_slots % 1000 + 7)
    T, W, H = 4, 2048, 64
    lens = np.array([2048, 1500, 333, 40], np.int32)
    table = _lists(rng, T, W, lens, num_slots, kv_dtype)
    live = np.unique(table[table >= 0]).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32) * 0.5)
    kv, pool = _pool(live, vals, num_slots, kv_dtype)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    atol = FP8_ATOL if kv_dtype == "fp8" else BF16_ATOL
    for splits in (0, 1):
        out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16,
                                           num_splits=splits)
        o = out.float().cpu().numpy()
        what = f"{kv_dtype} pool {num_slots} splits={splits}"
        gc.assert_close(o, o_ref, atol, BF16_RTOL, what + " out")
        gc.assert_lse(lse.cpu().numpy(), l_ref, LSE_ATOL, what + " lse")
        if kv_dtype == "bf16":
            assert gc.rel_l2(o, o_ref) <= 1e-2, (what, gc.rel_l2(o, o_ref))
    del kv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_slots", [(1 << 32) // 1152, 4_000_000])
def test_prefill_pool_at_4gib(num_slots):
    rng = np.random.default_rng(num_slots % 1000 + 11)
    Q, H, G, W = 6, 64, 2, 512
    lens = np.array([512, 400, 512, 77, 300, 512], np.int32)
    slots = _lists(rng, Q, W, lens, num_slots, "bf16")
    live = np.unique(slots[slots >= 0]).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * 0.5
    q = wl.f32_to_bf16_bits(rng.standard_normal((Q, H, 576)).astype(np.float32) * 0.5)
    kv, pool = _pool(live, vals, num_slots, "bf16")
    enc, ulens = smla.smla_build_group_union(_t(slots), _t(lens), G, num_slots)
    enc_o, lens_o = oracle.group_union(slots, lens, G, num_slots)
    enc_g, lens_g = enc.cpu().numpy().view(np.uint32), ulens.cpu().numpy()
    assert np.array_equal(lens_g, lens_o)
    for g in range(len(lens_o)):
        assert np.array_equal(enc_g[g, :lens_o[g]], enc_o[g, :lens_o[g]]), g
    out, lse = smla.smla_grouped_prefill(gc.q_tensor(q, "bf16"), kv, enc, ulens, G, 0.0625)
    o_ref, l_ref = oracle.grouped_prefill(q, pool, enc_o, lens_o, G, 0.0625)
    o = out.float().cpu().numpy()
    gc.assert_close(o, o_ref, BF16_ATOL, BF16_RTOL, f"prefill pool {num_slots}")
    gc.assert_lse(lse.cpu().numpy(), l_ref, LSE_ATOL, f"prefill pool {num_slots} lse")
    assert gc.rel_l2(o, o_ref) <= 1e-2
    del kv
    torch.cuda.empty_cache()
