"""Split decode on the GPU against the fp64 oracle (tolerances: bf16 |d| <= 2e-2 + 1e-2|ref|,
LSE |d| <= 1e-3, fp8 cache |d| <= 6e-2 + 1e-2|ref|; the fp32 path additionally 1e-4; every
bf16 case also a norm-relative error <= 1e-2). Unused pool slots hold NaN, so a wrong gather
cannot pass."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")

BF16_ATOL, BF16_RTOL, LSE_ATOL, FP8_ATOL = 2e-2, 1e-2, 1e-3, 6e-2


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(out, lse, o_ref, l_ref, atol, rtol, what, f32=False):
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    gc.assert_close(out, o_ref, atol, rtol, what + " out")
    gc.assert_lse(lse, l_ref, LSE_ATOL, what + " lse")
    if f32:
        gc.assert_close(out, o_ref, 1e-4, 0, what + " out (fp32 path)")
        gc.assert_lse(lse, l_ref, 1e-4, what + " lse (fp32 path)")
    else:
        assert gc.rel_l2(out, o_ref) <= 1e-2, (what, gc.rel_l2(out, o_ref))


def _random_case(seed, T, W, lens, num_slots, P=1, kv_dtype="bf16"):
    """Small decode case: T tokens, a NaN pool with rows only where tables point."""
    rng = np.random.default_rng(seed)
    H = 64
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32) * 0.5)
    if P == 1:
        table = np.full((T, W), -1, np.int32)
        for t in range(T):
            n = min(lens[t], W)
            table[t, :n] = rng.choice(num_slots, size=n, replace=False)
            if n > 4:
                table[t, rng.integers(0, n)] = -1      # a hole inside the valid prefix
        live = np.unique(table[table >= 0])
    else:
        pages = num_slots // P
        table = np.stack([rng.permutation(pages)[:W] for _ in range(T)]).astype(np.int32)
        live = np.unique(np.concatenate([table[t, :(-(-lens[t] // P))] for t in range(T)] + [np.zeros(0, np.int32)]))
        live = (live[:, None] * P + np.arange(P)[None, :]).reshape(-1)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    return q, table, np.asarray(lens, np.int32), live.astype(np.int32), vals


def _pools(live, vals, num_slots, kv_dtype):
    kv = smla.KvCache.empty(gc.KV_CODE[kv_dtype], num_slots)
    src = vals if kv_dtype != "bf16" else wl.f32_to_bf16_bits(vals)
    st, sd = gc.src_tensor(src)
    smla.smla_kv_write(st, _t(live), kv)
    pool = oracle.Pool(num_slots, kv_dtype)
    oracle.kv_write(pool, src, sd, live)
    return kv, pool


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [0, 1, 3, 8])
def test_decode_small_sparse(kv_dtype, splits):
    lens = [0, 1, 17, 31, 32, 33, 300, 2048]
    q, table, lens, live, vals = _random_case(11, len(lens), 2048, lens, 50000, kv_dtype=kv_dtype)
    kv, pool = _pools(live, vals, 50000, kv_dtype)
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16, num_splits=splits)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    atol = FP8_ATOL if kv_dtype == "fp8" else BF16_ATOL
    _check(out, lse, o_ref, l_ref, atol, BF16_RTOL, f"small {kv_dtype} splits={splits}")
    empty = lens == 0
    assert torch.all(out[torch.from_numpy(empty)] == 0)


@pytest.mark.parametrize("T,want_splits", [(1, 32), (2, 32), (4, 16)])
def test_decode_fp8_small_batch_plan(T, want_splits):
    """An fp8 cache at top-k 2048 under the automatic plan: 64-row splits at batch 1 and 2,
    128-row splits at batch 4 (the plan's floor), each against the oracle. Lengths cover a
    full list, a ragged tail and a list shorter than one split."""
    lens = [2048, 1000, 50, 2047][:T]
    q, table, lens, live, vals = _random_case(40 + T, T, 2048, lens, 30000, kv_dtype="fp8")
    kv, pool = _pools(live, vals, 30000, "fp8")
    qt = gc.q_tensor(q, "bf16")
    assert smla.smla_sparse_decode_splits(qt, kv, _t(table), _t(lens), 1, 1 / 16) == want_splits
    out, lse = smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), 1, 1 / 16)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    _check(out, lse, o_ref, l_ref, FP8_ATOL, BF16_RTOL, f"fp8 T={T} auto splits")


@pytest.mark.parametrize("P", [16, 64])
def test_decode_small_dense_paged(P):
    lens = [1, 63, 64, 65, 1000, 4000]
    q, table, lens, live, vals = _random_case(12 + P, len(lens), 4096 // P, lens, 8192, P=P)
    kv, pool = _pools(live, vals, 8192, "bf16")
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), P, 0.07)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, P, 0.07)
    _check(out, lse, o_ref, l_ref, BF16_ATOL, BF16_RTOL, f"dense P={P}")


def test_virtual_table_equals_page_table():
    """The same rows in the same order through resolved slots (page size 1) and through the
    page table (page size 64) give bitwise equal outputs."""
    P, T = 64, 4
    lens = np.array([100, 700, 2048, 64], np.int32)
    q, table, lens, live, vals = _random_case(13, T, 2048 // P, lens, 8192, P=P)
    kv, _ = _pools(live, vals, 8192, "bf16")
    qt = gc.q_tensor(q, "bf16")
    a = smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), P, 1 / 16, num_splits=4)
    pos = np.tile(np.arange(2048, dtype=np.int32), (T, 1))
    slots = smla.smla_resolve_slots(_t(pos), _t(lens), _t(np.arange(T, dtype=np.int32)), _t(table), _t(lens), P)
    b = smla.smla_sparse_decode(qt, kv, slots, _t(lens), 1, 1 / 16, num_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_deterministic():
    lens = [2048, 1500, 7]
    q, table, lens, live, vals = _random_case(14, 3, 2048, lens, 40000)
    kv, _ = _pools(live, vals, 40000, "bf16")
    qt = gc.q_tensor(q, "bf16")
    a = smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), 1, 1 / 16)
    b = smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), 1, 1 / 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _run_config(c):
    lay = c.layout
    kv, smap = gc.gpu_pool(smla, lay, c.rows, c.kv_dtype)
    pool, osl = gc.oracle_pool(lay, c.rows, c.kv_dtype)
    assert np.array_equal(smap.cpu().numpy(), osl)
    qt = gc.q_tensor(c.q, c.q_dtype)
    slots = smla.smla_resolve_slots(_t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx),
                                    lay.page_size)
    oslots = oracle.resolve_slots(c.idx, c.valid, c.tok_req, lay.page_table, lay.ctx, lay.page_size)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    sparse = np.setdiff1d(np.arange(len(c.idx)), c.dense_tokens)
    out, lse = smla.smla_sparse_decode(qt, kv, slots, _t(c.valid), 1, c.scale)
    o_ref, l_ref = oracle.sparse_decode(c.q, c.q_dtype, pool, oslots, c.valid, 1, c.scale, tokens=sparse)
    results = [(out[torch.from_numpy(sparse).cuda()], lse[torch.from_numpy(sparse).cuda()], o_ref, l_ref, "sparse rows")]
    if len(c.dense_tokens):
        d = c.dense_tokens
        dt = torch.from_numpy(d).cuda()
        pt_rows = lay.page_table[c.tok_req[d]]
        ctx = lay.ctx[c.tok_req[d]]
        out_d, lse_d = smla.smla_sparse_decode(qt[dt], kv, _t(pt_rows), _t(ctx), lay.page_size, c.scale)
        od, ld = oracle.sparse_decode(c.q[d], c.q_dtype, pool, pt_rows, ctx, lay.page_size, c.scale)
        results.append((out_d, lse_d, od, ld, "dense rows"))
    return results


def test_decode_tiny_f32_tiny_fp32():
    c = gc.config("decode_tiny_f32")
    for out, lse, o, l, what in _run_config(c):
        _check(out, lse, o, l, BF16_ATOL, BF16_RTOL, "decode_tiny_f32 " + what, f32=True)


def test_decode_bf16_b32_bf16():
    c = gc.config("decode_bf16_b32")
    for out, lse, o, l, what in _run_config(c):
        _check(out, lse, o, l, BF16_ATOL, BF16_RTOL, "decode_bf16_b32 " + what)


def test_decode_ragged_b128_ragged():
    c = gc.config("decode_ragged_b128")
    res = _run_config(c)
    assert len(res) == 2
    for out, lse, o, l, what in res:
        _check(out, lse, o, l, BF16_ATOL, BF16_RTOL, "decode_ragged_b128 " + what)


def test_decode_fp8_b64_fp8():
    c = gc.config("decode_fp8_b64")
    for out, lse, o, l, what in _run_config(c):
        _check(out, lse, o, l, FP8_ATOL, BF16_RTOL, "decode_fp8_b64 " + what)


def test_decode_graph_replay():
    """resolve + decode captured in a HIP graph; every replay matches the eager result."""
    c = wl.decode_bf16_b32(T=8)
    lay = c.layout
    kv, _ = gc.gpu_pool(smla, lay, c.rows, "bf16")
    qt = gc.q_tensor(c.q, "bf16")
    idx, valid, req = _t(c.idx), _t(c.valid), _t(c.tok_req)
    pt, ctx = _t(lay.page_table), _t(lay.ctx)
    slots = torch.empty_like(idx)
    out = torch.empty((8, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((8, 64), dtype=torch.float32, device="cuda")
    ws = smla.new_workspace(smla.smla_sparse_decode_workspace(qt, kv, idx, valid, 1, c.scale), "cuda")

    def step():
        smla.smla_resolve_slots(idx, valid, req, pt, ctx, lay.page_size, slots=slots)
        smla.smla_sparse_decode(qt, kv, slots, valid, 1, c.scale, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        assert int(ws[:256 * 1024].count_nonzero()) == 0, "merge counters not returned to zero by a replay"


@pytest.mark.parametrize("name", ["decode_bf16_b32", "decode_fp8_b64"])
def test_topk_fused_graph_replay(name):
    """The one-kernel step the benchmark times (top-k positions resolved inside stage 1, the
    splits merged inside it) captured twice into one HIP graph: every replay, with eager work
    and synchronisation between replays, equals the eager result bit for bit and leaves the
    merge counters at zero."""
    c = gc.config(name)
    lay = c.layout
    fmt = "fp8" if "fp8" in name else "bf16"
    kv, _ = gc.gpu_pool(smla, lay, c.rows, fmt)
    qt = gc.q_tensor(c.q, c.q_dtype)
    T, H = c.q.shape[0], c.q.shape[1]
    args = (_t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx), lay.page_size, c.scale)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = smla.new_workspace(smla.smla_sparse_decode_workspace(qt, kv, args[0], args[1], 1, c.scale), "cuda")

    def step():
        smla.smla_sparse_decode_topk(qt, kv, *args, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
        step()
    for _ in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        assert int(ws[:256 * 1024].count_nonzero()) == 0, "merge counters not returned to zero by a replay"


@pytest.mark.parametrize("name", ["decode_bf16_b32", "decode_ragged_b128", "decode_fp8_b64"])
def test_topk_fused_equals_resolve_then_decode(name):
    """smla_sparse_decode_topk (resolution inside stage 1) is bitwise smla_resolve_slots followed
    by the page size 1 decode, on the workloads' own index lists and page tables."""
    c = gc.config(name)
    lay = c.layout
    kv, _ = gc.gpu_pool(smla, lay, c.rows, c.kv_dtype)
    qt = gc.q_tensor(c.q, c.q_dtype)
    idx, valid, req, pt, ctx = _t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx)
    slots = smla.smla_resolve_slots(idx, valid, req, pt, ctx, lay.page_size)
    a = smla.smla_sparse_decode(qt, kv, slots, valid, 1, c.scale)
    b = smla.smla_sparse_decode_topk(qt, kv, idx, valid, req, pt, ctx, lay.page_size, c.scale)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("splits", [0, 3])
def test_topk_fused_masks(splits):
    """Every masking rule of slot resolution inside the fused path: invalid requests, negative
    positions, positions at or past the context, pages past the table row, page ids < 0,
    padding past the valid count, and an empty context."""
    rng = np.random.default_rng(21)
    T, W, R, P, ptw, pages = 6, 300, 4, 16, 20, 160
    num_slots = pages * P
    page_table = np.stack([rng.permutation(pages)[:ptw] for _ in range(R)]).astype(np.int32)
    page_table[1, 3] = -1
    page_table[3, [0, 7]] = -1
    seq_lens = np.array([320, 100, 0, 250], np.int32)
    tok_req = np.array([0, 1, 2, 3, 7, -1], np.int32)
    idx = np.stack([rng.choice(np.arange(-5, 340), size=W, replace=False) for _ in range(T)]).astype(np.int32)
    valid = np.array([300, 150, 300, 0, 300, 280], np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 64, 576)).astype(np.float32) * 0.5)
    live = np.arange(num_slots, dtype=np.int32)
    vals = rng.standard_normal((num_slots, 576)).astype(np.float32) * 0.5
    kv, pool = _pools(live, vals, num_slots, "bf16")
    qt = gc.q_tensor(q, "bf16")
    args = (_t(idx), _t(valid), _t(tok_req), _t(page_table), _t(seq_lens))
    slots = smla.smla_resolve_slots(*args, P)
    a = smla.smla_sparse_decode(qt, kv, slots, _t(valid), 1, 1 / 16, num_splits=splits)
    b = smla.smla_sparse_decode_topk(qt, kv, *args, P, 1 / 16, num_splits=splits)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oslots = oracle.resolve_slots(idx, valid, tok_req, page_table, seq_lens, P)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, oslots, valid, 1, 1 / 16)
    _check(b[0], b[1], o_ref, l_ref, BF16_ATOL, BF16_RTOL, f"fused masks splits={splits}")
    assert int((oslots >= 0).sum(axis=1).min()) == 0 and int((oslots >= 0).sum(axis=1).max()) > 100



@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_topk_requests_out_of_order(kv_dtype):
    """Tokens whose requests are not their own indices (a decode batch usually holds one token
    per request, in order, and stage 1 fetches request t's page-table row for token t before it
    knows the request): permuted and repeated requests through short page-table rows, tokens 1
    and 3 in their own index's request, tokens 5 and 6 past the last request index; the fused
    path against resolve + decode and the oracle."""
    rng = np.random.default_rng(41)
    T, W, R, P, ptw, pages = 7, 512, 5, 16, 40, 300
    num_slots = pages * P
    page_table = np.stack([rng.permutation(pages)[:ptw] for _ in range(R)]).astype(np.int32)
    seq_lens = np.array([600, 640, 333, 500, 17], np.int32)
    tok_req = np.array([3, 1, 4, 3, 1, 2, 0], np.int32)
    idx = np.stack([rng.choice(640, size=W, replace=False) for _ in range(T)]).astype(np.int32)
    valid = np.array([512, 400, 512, 512, 100, 512, 512], np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 64, 576)).astype(np.float32) * 0.5)
    live = np.arange(num_slots, dtype=np.int32)
    vals = rng.standard_normal((num_slots, 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    kv, pool = _pools(live, vals, num_slots, kv_dtype)
    qt = gc.q_tensor(q, "bf16")
    args = (_t(idx), _t(valid), _t(tok_req), _t(page_table), _t(seq_lens))
    slots = smla.smla_resolve_slots(*args, P)
    oslots = oracle.resolve_slots(idx, valid, tok_req, page_table, seq_lens, P)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    for splits in (0, 1):
        a = smla.smla_sparse_decode(qt, kv, slots, _t(valid), 1, 1 / 16, num_splits=splits)
        b = smla.smla_sparse_decode_topk(qt, kv, *args, P, 1 / 16, num_splits=splits)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, oslots, valid, 1, 1 / 16)
        atol = FP8_ATOL if kv_dtype == "fp8" else BF16_ATOL
        _check(b[0], b[1], o_ref, l_ref, atol, BF16_RTOL, f"requests out of order {kv_dtype} splits={splits}")


def test_topk_slots_past_int32():
    """Page ids whose slots pass the int32 range (page size 2^20; page id 4096 gives 2^32 + offset,
    which a 32-bit slot would wrap onto a slot inside the pool): smla_resolve_slots masks them
    as the oracle does, the fused path masks them too, and the two forms agree bitwise."""
    rng = np.random.default_rng(23)
    T, W, P, num_slots = 3, 512, 1 << 20, 1 << 16
    page_table = np.array([[0, 4096, 2048]], np.int32)
    seq_lens = np.array([3 * P], np.int32)
    tok_req = np.zeros(T, np.int32)
    idx = np.stack([np.concatenate([rng.choice(num_slots, W // 2, replace=False),
                                    P + rng.choice(num_slots, W // 4, replace=False),
                                    2 * P + rng.choice(num_slots, W // 4, replace=False)])
                    for _ in range(T)]).astype(np.int32)
    for t in range(T):
        rng.shuffle(idx[t])
    valid = np.full(T, W, np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 64, 576)).astype(np.float32) * 0.5)
    live = np.arange(num_slots, dtype=np.int32)
    vals = rng.standard_normal((num_slots, 576)).astype(np.float32) * 0.5
    kv, pool = _pools(live, vals, num_slots, "bf16")
    qt = gc.q_tensor(q, "bf16")
    args = (_t(idx), _t(valid), _t(tok_req), _t(page_table), _t(seq_lens))
    slots = smla.smla_resolve_slots(*args, P)
    oslots = oracle.resolve_slots(idx, valid, tok_req, page_table, seq_lens, P)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    assert int((oslots >= 0).sum()) == T * W // 2               # only the page-0 positions resolve
    a = smla.smla_sparse_decode(qt, kv, slots, _t(valid), 1, 1 / 16)
    b = smla.smla_sparse_decode_topk(qt, kv, *args, P, 1 / 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, oslots, valid, 1, 1 / 16)
    _check(b[0], b[1], o_ref, l_ref, BF16_ATOL, BF16_RTOL, "slots past int32")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_topk_long_page_table_row(kv_dtype):
    """A page-table row longer than the staging the fused path gives it in LDS (page size 1
    rows of 12000 / 6000 entries): each thread fetches the page ids of its own positions."""
    rng = np.random.default_rng(31)
    T, W, R, P = 4, 2048, 2, 1
    ptw = 12000 if kv_dtype == "bf16" else 6000
    pages = ptw + 500
    num_slots = pages * P
    page_table = np.stack([rng.permutation(pages)[:ptw] for _ in range(R)]).astype(np.int32)
    page_table[0, 5] = -1
    seq_lens = np.array([ptw - 37, ptw], np.int32)
    tok_req = np.array([0, 1, 0, 1], np.int32)
    idx = np.stack([rng.choice(ptw + 50, size=W, replace=False) - 10 for _ in range(T)]).astype(np.int32)
    idx[0, :3] = 5                                             # the page id < 0
    valid = np.array([2048, 2000, 1500, 2048], np.int32)
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 64, 576)).astype(np.float32) * 0.5)
    live = np.arange(num_slots, dtype=np.int32)
    vals = rng.standard_normal((num_slots, 576)).astype(np.float32) * (1.0 if kv_dtype == "fp8" else 0.5)
    kv, pool = _pools(live, vals, num_slots, kv_dtype)
    qt = gc.q_tensor(q, "bf16")
    args = (_t(idx), _t(valid), _t(tok_req), _t(page_table), _t(seq_lens))
    slots = smla.smla_resolve_slots(*args, P)
    a = smla.smla_sparse_decode(qt, kv, slots, _t(valid), 1, 1 / 16, num_splits=4)
    b = smla.smla_sparse_decode_topk(qt, kv, *args, P, 1 / 16, num_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oslots = oracle.resolve_slots(idx, valid, tok_req, page_table, seq_lens, P)
    assert np.array_equal(slots.cpu().numpy(), oslots)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, oslots, valid, 1, 1 / 16)
    atol = FP8_ATOL if kv_dtype == "fp8" else BF16_ATOL
    _check(b[0], b[1], o_ref, l_ref, atol, BF16_RTOL, f"long page-table row {kv_dtype}")

def _ws_counters(ws):
    return ws[:256 * 1024]


def test_merge_counters_return_to_zero_and_workspace_reuse():
    """The splits of a token merge inside stage 1 through counters at the head of the
    workspace: each call leaves them zero, so one workspace serves calls of different
    shapes one after another."""
    cases = []
    for seed, lens, splits in ((21, [2048, 900, 33, 1, 0, 1500, 64, 2048], 8), (22, [700, 2048, 5], 3)):
        q, table, lens, live, vals = _random_case(seed, len(lens), 2048, lens, 30000)
        cases.append((q, table, lens, live, vals, splits))
    need = max(smla.smla_sparse_decode_workspace(gc.q_tensor(c[0], "bf16"), smla.KvCache.empty(smla.SMLA_BF16, 8),
                                                 _t(c[1]), _t(c[2]), 1, 1 / 16, num_splits=c[5]) for c in cases)
    ws = smla.new_workspace(need, "cuda")
    for rep in range(2):
        for q, table, lens, live, vals, splits in cases:
            kv, pool = _pools(live, vals, 30000, "bf16")
            out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16,
                                               num_splits=splits, workspace=ws)
            torch.cuda.synchronize()
            assert int(_ws_counters(ws).count_nonzero()) == 0, "merge counters not returned to zero"
            o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
            _check(out, lse, o_ref, l_ref, BF16_ATOL, BF16_RTOL, f"reuse rep={rep} splits={splits}")


def test_merge_when_grid_exceeds_device():
    """More (token, split) workgroups than compute units: no workgroup waits for another,
    the last of each token to finish merges its splits."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = 8
    T = cus // splits + 9
    lens = [2048 - 37 * (t % 11) for t in range(T)]
    q, table, lens, live, vals = _random_case(23, T, 2048, lens, 200000)
    kv, pool = _pools(live, vals, 200000, "bf16")
    assert T * splits > cus
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16, num_splits=splits)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    _check(out, lse, o_ref, l_ref, BF16_ATOL, BF16_RTOL, "grid larger than the device")


def test_workspace_init_clears_counters():
    lens = [2048, 1000, 3]
    q, table, lens, live, vals = _random_case(24, 3, 2048, lens, 30000)
    kv, pool = _pools(live, vals, 30000, "bf16")
    qt = gc.q_tensor(q, "bf16")
    need = smla.smla_sparse_decode_workspace(qt, kv, _t(table), _t(lens), 1, 1 / 16, num_splits=4)
    ws = torch.full((need,), 0x5a, dtype=torch.uint8, device="cuda")
    smla.smla_sparse_decode_workspace_init(ws)
    out, lse = smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), 1, 1 / 16, num_splits=4, workspace=ws)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, table, lens, 1, 1 / 16)
    _check(out, lse, o_ref, l_ref, BF16_ATOL, BF16_RTOL, "initialised workspace")


@pytest.mark.parametrize("T", [4096, 4097])
def test_merge_in_stage2_past_counter_region(T):
    """The counter words cover 4,096 tokens. At 4,096 stage 1 still merges (the last token
    uses the last word); one token more and stage 2 merges the splits. A sample of tokens,
    the first and last of each region among them, against the oracle."""
    rng = np.random.default_rng(25)
    lens = rng.integers(1100, 2049, T)
    q, table, lens, live, vals = _random_case(25, T, 2048, lens, 30000)
    kv, pool = _pools(live, vals, 30000, "bf16")
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(table), _t(lens), 1, 1 / 16, num_splits=2)
    sample = [i for i in (0, 1, 2047, 4095, 4096) if i < T]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, table[sample], lens[sample], 1, 1 / 16)
    _check(out[sample], lse[sample], o_ref, l_ref, BF16_ATOL, BF16_RTOL, f"merge at T={T}")


def test_merge_bits_independent_of_arrival_order():
    """With more workgroups than compute units the merge parts fall to whichever workgroups
    arrive when, one part at a time or a head quarter's two halves together: the bits must
    not depend on it. Five repeats of a 32-token, 16-split decode (512 workgroups) agree."""
    rng = np.random.default_rng(26)
    lens = rng.integers(200, 2049, 32)
    q, table, lens, live, vals = _random_case(26, 32, 2048, lens, 60000)
    kv, pool = _pools(live, vals, 60000, "bf16")
    qt = gc.q_tensor(q, "bf16")
    runs = [smla.smla_sparse_decode(qt, kv, _t(table), _t(lens), 1, 0.1, num_splits=16) for _ in range(5)]
    for o, l in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])
    sample = [0, 17, 31]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, table[sample], lens[sample], 1, 0.1)
    _check(runs[0][0][sample], runs[0][1][sample], o_ref, l_ref, BF16_ATOL, BF16_RTOL, "arrival-order merge")


def _dense_case(seed, ctx, P, pool_extra=16):
    """Requests with contexts `ctx`, each with its own pages (dealt from a permutation), the
    slots of the pages a context covers written; q for 64 heads."""
    rng = np.random.default_rng(seed)
    T = len(ctx)
    ptw = max(1, -(-int(max(ctx)) // P))
    num_pages = T * ptw + pool_extra
    pt = rng.permutation(num_pages)[:T * ptw].reshape(T, ptw).astype(np.int32)
    used = np.concatenate([pt[t, :-(-int(c) // P)] for t, c in enumerate(ctx)] + [np.zeros(0, np.int32)])
    live = np.unique((used[:, None] * P + np.arange(P)[None, :]).reshape(-1)).astype(np.int32)
    vals = rng.standard_normal((len(live), 576)).astype(np.float32) * 0.5
    kv, pool = _pools(live, vals, num_pages * P, "bf16")
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 64, 576)).astype(np.float32) * 0.5)
    return q, pt, np.asarray(ctx, np.int32), kv, pool


@pytest.mark.parametrize("T", [64, 65])
def test_dense_paged_planned_splits(T):
    """Dense paged decode with contexts from 0 to 32K: up to 64 tokens plan their splits on
    the device from the lengths, 65 use the uniform plan; sampled tokens against the oracle."""
    rng = np.random.default_rng(27 + T)
    ctx = rng.integers(0, 8193, T)
    ctx[0], ctx[1], ctx[2] = 0, 32768, 1
    q, pt, ctx, kv, pool = _dense_case(27 + T, ctx, 64)
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(pt), _t(ctx), 64, 1 / 16)
    sample = [0, 1, 2, T // 2, T - 1]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, pt[sample], ctx[sample], 64, 1 / 16)
    _check(out[sample], lse[sample], o_ref, l_ref, BF16_ATOL, BF16_RTOL, f"dense planned T={T}")
    assert torch.all(out[0] == 0)


def test_dense_paged_planned_one_long_context():
    """One 64K context and one short one: the plan gives the long one about 220 splits (rows
    per split from the total), merged through one token word; the result against the oracle."""
    q, pt, ctx, kv, pool = _dense_case(28, [65536, 300], 64)
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(pt), _t(ctx), 64, 1 / 16)
    o_ref, l_ref = oracle.sparse_decode(q, "bf16", pool, pt, ctx, 64, 1 / 16)
    _check(out, lse, o_ref, l_ref, BF16_ATOL, BF16_RTOL, "dense planned 64K")


def test_dense_paged_planned_long_splits():
    """Eight contexts of 40K-64K (and one of 100): the balanced plan keeps one workgroup per
    compute unit, so each split holds more rows than one 1,024-row segment and walks them
    segment by segment (page ids copied per segment), with O, max and sum carried across;
    sampled tokens against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(29)
    ctx = [int(x) for x in rng.integers(40000, 65537, 8)] + [100]
    assert sum(ctx) > 1024 * cus                      # rows per split above one segment
    q, pt, ctx, kv, pool = _dense_case(29, ctx, 64)
    out, lse = smla.smla_sparse_decode(gc.q_tensor(q, "bf16"), kv, _t(pt), _t(ctx), 64, 1 / 16)
    sample = [0, 5, 8]
    o_ref, l_ref = oracle.sparse_decode(q[sample], "bf16", pool, pt[sample], ctx[sample], 64, 1 / 16)
    _check(out[sample], lse[sample], o_ref, l_ref, BF16_ATOL, BF16_RTOL, "dense planned long splits")
