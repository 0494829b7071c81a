"""Grouped prefill on the GPU against the oracle (bf16 tolerances as decode)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _small(seed, Q, H, G, W=256, ns=3000):
    rng = np.random.default_rng(seed)
    slots, valid = wl.random_slot_lists(seed, Q, W, ns, overlap=0.7, G=G, pad_frac=0.3)
    vals = wl.f32_to_bf16_bits(rng.standard_normal((ns, 576)).astype(np.float32) * 0.5)
    live = np.unique(slots[slots >= 0]).astype(np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((Q, H, 576)).astype(np.float32) * 0.5)
    kv = smla.KvCache.empty(smla.SMLA_BF16, ns)
    smla.smla_kv_write(gc.bits_to_torch_bf16(vals[live]), _t(live), kv)
    pool = oracle.Pool(ns, "bf16")
    oracle.kv_write(pool, vals[live], "bf16", live)
    return q, slots, valid, kv, pool, ns


@pytest.mark.parametrize("Q,H,G", [(9, 64, 2), (2, 64, 2), (10, 32, 4), (13, 16, 8)])
def test_prefill_small(Q, H, G):
    q, slots, valid, kv, pool, ns = _small(20 + Q + G, Q, H, G)
    enc, lens = smla.smla_build_group_union(_t(slots), _t(valid), G, ns)
    out, lse = smla.smla_grouped_prefill(gc.q_tensor(q, "bf16"), kv, enc, lens, G, 0.0625)
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    o_ref, l_ref = oracle.grouped_prefill(q, pool, enc_o, lens_o, G, 0.0625)
    # each query also equals decode over its own list
    od, ld = oracle.sparse_decode(q, "bf16", pool, slots, valid, 1, 0.0625)
    assert np.allclose(o_ref, od, atol=1e-12) and np.allclose(np.nan_to_num(l_ref, neginf=-1e300),
                                                              np.nan_to_num(ld, neginf=-1e300), atol=1e-12)
    o = out.float().cpu().numpy()
    gc.assert_close(o, o_ref, 2e-2, 1e-2, f"prefill Q={Q} G={G}")
    gc.assert_lse(lse.cpu().numpy(), l_ref, 1e-3, f"prefill Q={Q} G={G} lse")
    assert gc.rel_l2(o, o_ref) <= 1e-2
    # planted in the oracle, on the CPU: the second member's bit cleared, or the tail
    # query dropped, gives an expectation the GPU result must NOT meet
    if Q >= 2:
        bad = enc_o.copy()
        bad[:, :] &= ~np.uint32(1 << 25)
        ob, _ = oracle.grouped_prefill(q, pool, bad, lens_o, G, 0.0625, queries=[1])
        assert gc.rel_l2(o[1], ob[0]) > 0.05
    # the last query (the short last group's tail when Q % G != 0) dropped from its group
    tail, gl, m = Q - 1, (Q - 1) // G, (Q - 1) % G
    bad = enc_o.copy()
    bad[gl, :] &= ~np.uint32(1 << (24 + m))
    ob, lb = oracle.grouped_prefill(q, pool, bad, lens_o, G, 0.0625, queries=[tail])
    assert np.all(ob[0] == 0) and np.all(np.isneginf(lb[0]))
    assert gc.rel_l2(o[tail], ob[0]) > 0.05 and np.all(np.isfinite(lse[tail].cpu().numpy()))


def _fp8_pool(vals, live, ns):
    kv = smla.KvCache.empty(smla.SMLA_FP8_E4M3, ns)
    smla.smla_kv_write(_t(vals[live]), _t(live), kv)
    pool = oracle.Pool(ns, "fp8")
    oracle.kv_write(pool, vals[live], "f32", live)
    return kv, pool


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("H,G", [(64, 2), (32, 4), (16, 8)])
def test_prefill_long_union(kv_dtype, H, G):
    """Groups whose union spans several segments of the walk (little overlap), a member with
    an empty list next to full ones, a short last group, and an fp8 cache; with H < 64 one
    workgroup serves several members, each head masked by its own member's bit."""
    rng = np.random.default_rng(61 + H)
    Q, W, ns = 6, 2048 // G, 6000
    slots, valid = wl.random_slot_lists(61 + H, Q, W, ns, overlap=0.1, G=G)
    valid[3] = 0                                           # a member with no rows
    valid[4] = W - 37
    vals = rng.standard_normal((ns, 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    live = np.unique(slots[slots >= 0]).astype(np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((Q, H, 576)).astype(np.float32) * 0.5)
    if kv_dtype == "bf16":
        vb = wl.f32_to_bf16_bits(vals)
        kv = smla.KvCache.empty(smla.SMLA_BF16, ns)
        smla.smla_kv_write(gc.bits_to_torch_bf16(vb[live]), _t(live), kv)
        pool = oracle.Pool(ns, "bf16")
        oracle.kv_write(pool, vb[live], "bf16", live)
    else:
        kv, pool = _fp8_pool(vals, live, ns)
    enc, lens = smla.smla_build_group_union(_t(slots), _t(valid), G, ns)
    out, lse = smla.smla_grouped_prefill(gc.q_tensor(q, "bf16"), kv, enc, lens, G, 0.0625)
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    assert np.array_equal(lens.cpu().numpy(), lens_o) and int(lens_o.max()) > 1024   # more than one segment
    o_ref, l_ref = oracle.grouped_prefill(q, pool, enc_o, lens_o, G, 0.0625)
    o = out.float().cpu().numpy()
    atol = 6e-2 if kv_dtype == "fp8" else 2e-2
    gc.assert_close(o, o_ref, atol, 1e-2, f"prefill H={H} G={G} {kv_dtype}")
    gc.assert_lse(lse.cpu().numpy(), l_ref, 1e-3, f"prefill H={H} G={G} {kv_dtype} lse")
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3].cpu().numpy()))


def test_prefill_grouped_q8192_sampled():
    c = gc.config("prefill_grouped_q8192")
    lay = c.layout
    kv, smap = gc.gpu_pool(smla, lay, c.rows, "bf16")
    pool, osl = gc.oracle_pool(lay, c.rows, "bf16")
    req = np.zeros(len(c.idx), np.int32)
    slots = smla.smla_resolve_slots(_t(c.idx), _t(c.valid), _t(req), _t(lay.page_table), _t(lay.ctx), lay.page_size)
    oslots = oracle.resolve_slots(c.idx, c.valid, req, lay.page_table, lay.ctx, lay.page_size)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    enc, lens = smla.smla_build_group_union(slots, _t(c.valid), c.G, lay.num_slots)
    out, lse = smla.smla_grouped_prefill(gc.q_tensor(c.q, "bf16"), kv, enc, lens, c.G, c.scale)
    rng = np.random.default_rng(44)
    sample = np.sort(np.concatenate([rng.choice(np.arange(1, len(c.idx) - 1), size=1022, replace=False),
                                     [0, len(c.idx) - 1]]))
    enc_o, lens_o = oracle.group_union(oslots, c.valid, c.G, lay.num_slots)
    assert np.array_equal(lens.cpu().numpy(), lens_o)
    o_ref, l_ref = oracle.grouped_prefill(c.q, pool, enc_o, lens_o, c.G, c.scale, queries=sample)
    o = out[torch.from_numpy(sample).cuda()].float().cpu().numpy()
    gc.assert_close(o, o_ref, 2e-2, 1e-2, "prefill_grouped_q8192 out")
    gc.assert_lse(lse[torch.from_numpy(sample).cuda()].cpu().numpy(), l_ref, 1e-3, "prefill_grouped_q8192 lse")
    assert gc.rel_l2(o, o_ref) <= 1e-2


@pytest.mark.parametrize("Q,H,G", [(9, 64, 2), (13, 16, 8)])
def test_prefill_graph_replay(Q, H, G):
    """Union build + grouped prefill captured into a HIP graph: every replay, with eager work and
    synchronisation between replays, gives the eager union, lengths and outputs bit for bit."""
    q, slots, valid, kv, pool, ns = _small(40 + Q + G, Q, H, G)
    st, vt, qt = _t(slots), _t(valid), gc.q_tensor(q, "bf16")
    ng = -(-Q // G)
    enc = torch.empty((ng, G * slots.shape[1]), dtype=torch.int32, device="cuda")
    lens = torch.empty((ng,), dtype=torch.int32, device="cuda")
    out = torch.empty((Q, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Q, H), dtype=torch.float32, device="cuda")

    def step():
        smla.smla_build_group_union(st, vt, G, ns, enc=enc, lens=lens)
        smla.smla_grouped_prefill(qt, kv, enc, lens, G, 0.0625, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [lens.clone(), out.clone(), lse.clone()]
    ref_enc = [enc[g, :int(ref[0][g])].clone() for g in range(ng)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        enc.fill_(-7)
        lens.fill_(-1)
        out.fill_(float("nan"))
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lens, ref[0]) and torch.equal(out, ref[1]) and torch.equal(lse, ref[2])
        for k in range(ng):
            assert torch.equal(enc[k, :int(ref[0][k])], ref_enc[k])
    enc_o, lens_o = oracle.group_union(slots, valid, G, ns)
    assert np.array_equal(lens.cpu().numpy(), lens_o)
