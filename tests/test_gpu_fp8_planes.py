"""fp8 caches whose three planes (e4m3 codes, bf16 rotary part, fp32 scale) live in separate
tensors with padded strides, the general form of the fp8 cache descriptor. The cache write, the
split decode (over slots and with the top-k positions resolved in the kernel) and the grouped
prefill give the same bits as over the packed 656-byte rows, and match the fp64 oracle. Every
plane's padding and every unwritten slot hold NaN patterns, so a read outside a plane's own
bytes cannot pass."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")

FP8_ATOL, RTOL, LSE_ATOL = 6e-2, 1e-2, 1e-3
LAT_STRIDE, ROPE_STRIDE, SCALE_STRIDE = 528, 144, 8      # bytes: 16 / 16 / 4 bytes of padding per slot


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class PlanarKv:
    """An fp8 pool as three separately allocated planes (same interface as smla.KvCache)."""

    def __init__(self, num_slots: int):
        self.dtype = smla.SMLA_FP8_E4M3
        self.num_slots = num_slots
        self.lat = torch.full((num_slots, LAT_STRIDE), 0x7F, dtype=torch.uint8, device="cuda")
        self.rope = torch.full((num_slots, ROPE_STRIDE // 2), 0x7FC0, dtype=torch.int16, device="cuda")
        self.sc = torch.full((num_slots, SCALE_STRIDE // 4), float("nan"), dtype=torch.float32, device="cuda")

    def desc(self):
        d = smla.smla.smla_kv()
        d.dtype = self.dtype
        d.num_slots = self.num_slots
        d.lat8, d.lat8_stride = self.lat.data_ptr(), LAT_STRIDE
        d.rope16, d.rope16_stride = self.rope.data_ptr(), ROPE_STRIDE
        d.scale, d.scale_stride = self.sc.data_ptr(), SCALE_STRIDE
        return d


def _pools(vals, live, ns):
    packed = smla.KvCache.empty(smla.SMLA_FP8_E4M3, ns, layout="packed")
    planar = PlanarKv(ns)
    src, sl = _t(vals[live]), _t(live)
    smla.smla_kv_write(src, sl, packed)
    smla.smla_kv_write(src, sl, planar)
    pool = oracle.Pool(ns, "fp8")
    oracle.kv_write(pool, vals[live], "f32", live)
    return packed, planar, pool


def test_fp8_planes_write():
    rng = np.random.default_rng(71)
    ns = 3000
    vals = rng.standard_normal((ns, 576)).astype(np.float32)
    vals[5] *= 1e-30                                      # a row of subnormal magnitudes
    vals[6] = 0.0                                         # an all-zero row
    live = np.sort(rng.choice(ns, 900, replace=False)).astype(np.int32)
    packed, planar, _ = _pools(vals, live, ns)
    lv = _t(live).long()
    assert torch.equal(planar.lat[lv, :512], packed.lat8()[lv])
    assert torch.equal(planar.rope[lv, :64], packed.rope16()[lv])
    assert torch.equal(planar.sc[lv, 0].view(torch.int32), packed.scale()[lv].view(torch.int32))
    # padding, and every slot the write did not name, keep their NaN patterns
    assert bool(torch.all(planar.lat[:, 512:] == 0x7F)) and bool(torch.all(planar.rope[:, 64:] == 0x7FC0))
    assert bool(torch.all(torch.isnan(planar.sc[:, 1])))
    dead = torch.ones(ns, dtype=torch.bool, device="cuda")
    dead[lv] = False
    assert bool(torch.all(planar.lat[dead] == 0x7F)) and bool(torch.all(torch.isnan(planar.sc[dead, 0])))


@pytest.mark.parametrize("splits", [0, 3])
def test_fp8_planes_decode(splits):
    rng = np.random.default_rng(72)
    lens = np.array([0, 1, 31, 33, 300, 1500, 2048, 700], np.int32)
    T, W, ns, H = len(lens), 2048, 40000, 64
    table = np.full((T, W), -1, np.int32)
    for t in range(T):
        table[t, :lens[t]] = rng.choice(ns, size=lens[t], replace=False)
    live = np.unique(table[table >= 0]).astype(np.int32)
    vals = rng.standard_normal((ns, 576)).astype(np.float32)
    packed, planar, pool = _pools(vals, live, ns)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32) * 0.5)
    qt = gc.q_tensor(q, "bf16")
    a = smla.smla_sparse_decode(qt, packed, _t(table), _t(lens), 1, 1 / 16, num_splits=splits)
    b = smla.smla_sparse_decode(qt, planar, _t(table), _t(lens), 1, 1 / 16, num_splits=splits)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    gc.assert_close(b[0].float().cpu().numpy(), o_ref, FP8_ATOL, RTOL, f"planar fp8 decode splits={splits}")
    gc.assert_lse(b[1].cpu().numpy(), l_ref, LSE_ATOL, f"planar fp8 decode splits={splits} lse")


def test_fp8_planes_decode_topk():
    """The fused top-k decode on the fp8 workload's own index lists and page tables."""
    c = gc.config("decode_fp8_b64")
    lay = c.layout
    packed, _ = gc.gpu_pool(smla, lay, c.rows, "fp8")
    planar = PlanarKv(packed.num_slots)
    planar.lat[:, :512].copy_(packed.lat8())
    planar.rope[:, :64].copy_(packed.rope16())
    planar.sc[:, 0].copy_(packed.scale())
    qt = gc.q_tensor(c.q, c.q_dtype)
    args = (_t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx), lay.page_size, c.scale)
    a = smla.smla_sparse_decode_topk(qt, packed, *args)
    b = smla.smla_sparse_decode_topk(qt, planar, *args)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_planes_prefill():
    rng = np.random.default_rng(73)
    H, G, Q, ns = 64, 2, 6, 6000
    W = 2048 // G
    slots, valid = wl.random_slot_lists(73, Q, W, ns, overlap=0.1, G=G)
    valid[4] = W - 37
    vals = rng.standard_normal((ns, 576)).astype(np.float32)
    live = np.unique(slots[slots >= 0]).astype(np.int32)
    packed, planar, pool = _pools(vals, live, ns)
    q = wl.f32_to_bf16_bits(rng.standard_normal((Q, H, 576)).astype(np.float32) * 0.5)
    qt = gc.q_tensor(q, "bf16")
    enc, lens = smla.smla_build_group_union(_t(slots), _t(valid), G, ns)
    a = smla.smla_grouped_prefill(qt, packed, enc, lens, G, 0.0625)
    b = smla.smla_grouped_prefill(qt, planar, enc, lens, G, 0.0625)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    o_ref, l_ref = oracle.grouped_prefill(q, pool, enc_o, lens_o, G, 0.0625)
    gc.assert_close(b[0].float().cpu().numpy(), o_ref, FP8_ATOL, RTOL, "planar fp8 prefill")
    gc.assert_lse(b[1].cpu().numpy(), l_ref, LSE_ATOL, "planar fp8 prefill lse")
