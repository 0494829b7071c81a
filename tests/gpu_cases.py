"""Build the same seeded inputs on both sides: the HIP path (through libsmla) and the CPU
oracle (through its own arithmetic). The only thing the two share is the generator output
from `workloads`; each side resolves slots and writes its cache by itself."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import workloads as wl

KV_CODE = {"f32": 0, "bf16": 1, "fp8": 2}


def bits_to_torch_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def q_tensor(q: np.ndarray, q_dtype: str, device="cuda") -> torch.Tensor:
    if q_dtype == "bf16":
        return bits_to_torch_bf16(q, device)
    return torch.from_numpy(np.ascontiguousarray(q)).to(device)


def src_tensor(values: np.ndarray, device="cuda") -> tuple[torch.Tensor, str]:
    if values.dtype == np.uint16:
        return bits_to_torch_bf16(values, device), "bf16"
    return torch.from_numpy(np.ascontiguousarray(values)).to(device), "f32"


def gpu_pool(smla, layout: wl.PagedLayout, rows: wl.LogicalRows, kv_dtype: str, device="cuda"):
    """NaN-poisoned pool in which the listed logical rows are written through
    smla_resolve_slots + smla_kv_write."""
    kv = smla.KvCache.empty(KV_CODE[kv_dtype], layout.num_slots, device=device, poison=True)
    pt = torch.from_numpy(layout.page_table).to(device)
    ctx = torch.from_numpy(layout.ctx).to(device)
    pos = torch.from_numpy(np.ascontiguousarray(rows.pos[:, None])).to(device)
    req = torch.from_numpy(rows.req).to(device)
    smap = smla.smla_resolve_slots(pos, None, req, pt, ctx, layout.page_size)[:, 0].contiguous()
    src, _ = src_tensor(rows.values, device)
    smla.smla_kv_write(src, smap, kv)
    return kv, smap


def oracle_pool(layout: wl.PagedLayout, rows: wl.LogicalRows, kv_dtype: str):
    pool = oracle.Pool(layout.num_slots, kv_dtype)
    sl = oracle.resolve_slots(rows.pos[:, None], None, rows.req, layout.page_table, layout.ctx,
                              layout.page_size)[:, 0]
    src_dtype = "bf16" if rows.values.dtype == np.uint16 else "f32"
    oracle.kv_write(pool, rows.values, src_dtype, sl)
    return pool, sl


def assert_close(got: np.ndarray, want: np.ndarray, atol: float, rtol: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert not np.any(np.isnan(got)), f"{what}: NaN in GPU output"
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = err > bound
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside |d| <= {atol} + {rtol}|ref|; "
                             f"worst at {i}: got {got[i]!r} want {want[i]!r}")


def assert_lse(got: np.ndarray, want: np.ndarray, atol: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    empty = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), empty), f"{what}: empty-set (-inf) pattern differs"
    if np.any(~empty):
        d = np.abs(got[~empty] - want[~empty])
        assert d.max() <= atol, f"{what}: max |dLSE| {d.max():.3g} > {atol}"


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


@functools.lru_cache(maxsize=None)
def config(name: str):
    """Generate a workload once per test session."""
    return getattr(wl, name)()
