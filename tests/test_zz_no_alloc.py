"""The allocation-free decode (smla_sparse_decode_noalloc: its workspace is the library's static
scratch array) against the entry points it mirrors, smla_sparse_decode_topk and
smla_sparse_decode, which take a caller workspace. Same kernels and split plan, so the outputs
must be equal bit for bit; two calls in a row, the second smaller, so that the second runs
over the scratch the first left behind."""
import numpy as np
import pytest
import torch

from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_equals_workspace_decode_twice():
    c = gc.config("decode_bf16_b32")
    lay = c.layout
    kv, _ = gc.gpu_pool(smla, lay, c.rows, c.kv_dtype)
    qt = gc.q_tensor(c.q, c.q_dtype)
    idx, valid, req, pt, ctx = _t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx)
    pm = (req, pt, ctx, lay.page_size)

    # first call: the whole batch of 32 tokens (8 splits each, merged inside stage 1)
    ref = smla.smla_sparse_decode_topk(qt, kv, idx, valid, req, pt, ctx, lay.page_size, c.scale)
    got = smla.smla_sparse_decode_noalloc(qt, kv, idx, valid, 1, c.scale, page_map=pm)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])

    # second call, smaller: 5 tokens (more splits each) with shorter valid counts, over the
    # scratch the first call left
    n = 5
    v2 = _t(np.array([2048, 1500, 700, 33, 0], np.int32))
    ref2 = smla.smla_sparse_decode_topk(qt[:n], kv, idx[:n], v2, req[:n], pt, ctx, lay.page_size, c.scale)
    got2 = smla.smla_sparse_decode_noalloc(qt[:n], kv, idx[:n], v2, 1, c.scale, page_map=(req[:n], pt, ctx,
                                                                                             lay.page_size))
    torch.cuda.synchronize()
    assert torch.equal(ref2[0], got2[0]) and torch.equal(ref2[1], got2[1])
    assert torch.all(got2[0][4] == 0) and torch.all(torch.isneginf(got2[1][4]))      # the empty token

    # the slot-table form (no page map), 3 tokens with 3 forced splits, then the merge words are
    # back at zero: a fourth call equals its workspace twin again
    slots = smla.smla_resolve_slots(idx, valid, req, pt, ctx, lay.page_size)
    ref3 = smla.smla_sparse_decode(qt[:3], kv, slots[:3], valid[:3], 1, c.scale, num_splits=3)
    got3 = smla.smla_sparse_decode_noalloc(qt[:3], kv, slots[:3], valid[:3], 1, c.scale, num_splits=3)
    got4 = smla.smla_sparse_decode_noalloc(qt, kv, idx, valid, 1, c.scale, page_map=pm)
    torch.cuda.synchronize()
    assert torch.equal(ref3[0], got3[0]) and torch.equal(ref3[1], got3[1])
    assert torch.equal(ref[0], got4[0]) and torch.equal(ref[1], got4[1])


def test_noalloc_fp8_cache():
    """The fp8-cache decode (batch 64, 4 splits) through the static scratch equals its
    workspace twin."""
    c = gc.config("decode_fp8_b64")
    lay = c.layout
    kv, _ = gc.gpu_pool(smla, lay, c.rows, c.kv_dtype)
    qt = gc.q_tensor(c.q, c.q_dtype)
    idx, valid, req, pt, ctx = _t(c.idx), _t(c.valid), _t(c.tok_req), _t(lay.page_table), _t(lay.ctx)
    ref = smla.smla_sparse_decode_topk(qt, kv, idx, valid, req, pt, ctx, lay.page_size, c.scale)
    got = smla.smla_sparse_decode_noalloc(qt, kv, idx, valid, 1, c.scale, page_map=(req, pt, ctx, lay.page_size))
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
