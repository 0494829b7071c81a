"""Cache writes on the GPU against the oracle's cache write: stored bits must be equal."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from . import gpu_cases as gc

pytestmark = pytest.mark.gpu
smla = pytest.importorskip("sparse_mla_attention_resolve_amd")


def _src(rng, n, src_dtype):
    x = rng.standard_normal((n, 576)).astype(np.float32) * rng.choice([1e-3, 1.0, 40.0], size=(n, 1)).astype(np.float32)
    x[0, :512] = 0.0                              # zero latent -> scale 0, codes 0
    x[1, 7] = 3e4                                 # one huge element
    x[2, :512] = 2.0 ** -20                       # tiny values
    x[3, 100] = -x[3, :512].__abs__().max() * 3   # negative amax
    if src_dtype == "bf16":
        return wl.f32_to_bf16_bits(x)
    return x


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("src_dtype", ["f32", "bf16"])
def test_kv_write_bits(kv_dtype, src_dtype):
    rng = np.random.default_rng(hash((kv_dtype, src_dtype)) % 1000)
    n, ns = 300, 1000
    src = _src(rng, n, src_dtype)
    smap = rng.choice(ns, size=n, replace=False).astype(np.int32)
    smap[5] = -1
    smap[6] = ns + 10                             # past the pool: skipped
    kv = smla.KvCache.empty(gc.KV_CODE[kv_dtype], ns)
    st, _ = gc.src_tensor(src)
    smla.smla_kv_write(st, torch.from_numpy(smap).cuda(), kv)
    pool = oracle.Pool(ns, kv_dtype)
    keep = (smap >= 0) & (smap < ns)
    oracle.kv_write(pool, src[keep], src_dtype, smap[keep])
    written = smap[keep]
    want = pool.stored(written)
    stor = kv.storage.cpu()
    if kv_dtype == "f32":
        got = stor.numpy()[written]
        assert np.array_equal(got.view(np.uint32), want["rows"].view(np.uint32))
    elif kv_dtype == "bf16":
        got = stor.view(torch.int16).numpy().view(np.uint16)[written]
        assert np.array_equal(got, want["rows"])
    else:
        w = torch.from_numpy(written).cuda()
        assert np.array_equal(kv.lat8()[w].cpu().numpy(), want["lat8"])
        assert np.array_equal(kv.rope16()[w].cpu().numpy().view(np.uint16), want["rope16"])
        assert np.array_equal(kv.scale()[w].cpu().numpy().view(np.uint32), want["scale"].view(np.uint32))
    # every other slot still holds the poison
    others = np.setdiff1d(np.arange(ns), written)
    if kv_dtype == "fp8":
        o = torch.from_numpy(others).cuda()
        assert bool((kv.lat8()[o] == 0x7F).all()) and bool(torch.isnan(kv.scale()[o]).all())
    else:
        assert torch.isnan(stor[torch.from_numpy(others)].float()).all()


def test_kv_write_fp8_b64_codes():
    c = wl.decode_fp8_b64(T=8)
    kv, smap = gc.gpu_pool(smla, c.layout, c.rows, "fp8")
    pool, osl = gc.oracle_pool(c.layout, c.rows, "fp8")
    assert np.array_equal(smap.cpu().numpy(), osl)
    sl = smap.long()
    want = pool.stored(osl)
    assert np.array_equal(kv.lat8()[sl].cpu().numpy(), want["lat8"])
    assert np.array_equal(kv.rope16()[sl].cpu().numpy().view(np.uint16), want["rope16"])
    assert np.array_equal(kv.scale()[sl].cpu().numpy(), want["scale"])


def _e4m3_values():
    """Every e4m3 value, and for each pair of neighbours their exact midpoint (a tie) and the
    fp32 values one step either side of it, both signs, plus zeros and the saturation edge."""
    mags = [0.0]
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                           # 0x7f is NaN
            mags.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    mags = np.array(sorted(set(mags)), np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                           mags.astype(np.float32), np.float32([448.0, np.nextafter(np.float32(448), np.float32(0))])])
    vals = np.concatenate([near, -near, np.float32([0.0, -0.0, 1e-45, -1e-45, 2.0 ** -130])]).astype(np.float32)
    return vals


def test_kv_write_fp8_rounding_edges():
    """The stored e4m3 codes of values at and around every rounding midpoint (ties to even),
    subnormals, signed zeros and the top of the range equal the reference encoder's. A row
    whose latent amax is 448 has scale 1, so its codes are the encodings of the values."""
    vals = _e4m3_values()
    per = 511
    n = -(-len(vals) // per)
    src = np.zeros((n, 576), np.float32)
    src[:, 0] = 448.0
    flat = np.zeros(n * per, np.float32)
    flat[:len(vals)] = vals
    src[:, 1:512] = flat.reshape(n, per)
    ns = n + 3
    smap = np.arange(n, dtype=np.int32) + 1
    kv = smla.KvCache.empty(smla.SMLA_FP8_E4M3, ns)
    smla.smla_kv_write(torch.from_numpy(src).cuda(), torch.from_numpy(smap).cuda(), kv)
    pool = oracle.Pool(ns, "fp8")
    oracle.kv_write(pool, src, "f32", smap)
    want = pool.stored(smap)
    s = kv.storage.cpu().numpy()[smap]
    assert np.all(want["scale"] == np.float32(1.0))
    assert np.array_equal(s[:, :512], want["lat8"])


def test_kv_write_fp8_nonfinite_rows():
    """Rows holding a NaN or an infinity. The maximum over a latent row that holds a NaN is
    NaN, so its scale is NaN and all 512 codes are the NaN code; a NaN in the rotary part
    leaves the scale alone. A latent infinity gives an infinite scale: finite values encode
    to signed zeros and the infinity itself to the NaN code (inf / inf). Codes equal the
    oracle's bit for bit; scales equal it bit for bit where finite, and are NaN together."""
    rng = np.random.default_rng(7)
    src = rng.standard_normal((8, 576)).astype(np.float32)
    src[0, 0] = np.nan
    src[1, 511] = np.nan
    src[2, 300] = -np.nan
    src[3, 520] = np.nan          # rotary column only
    src[4, 17] = np.inf
    src[5, 400] = -np.inf
    src[6, :512] = 0.0            # all-zero latent: scale 0, codes 0
    smap = np.arange(8, dtype=np.int32) * 3 + 2
    ns = 8 * 3 + 2
    kv = smla.KvCache.empty(smla.SMLA_FP8_E4M3, ns)
    smla.smla_kv_write(torch.from_numpy(src).cuda(), torch.from_numpy(smap).cuda(), kv)
    pool = oracle.Pool(ns, "fp8")
    oracle.kv_write(pool, src, "f32", smap)
    want = pool.stored(smap)
    got_codes = kv.lat8()[torch.from_numpy(smap).long()].cpu().numpy()
    got_scale = kv.scale()[torch.from_numpy(smap).long()].cpu().numpy()
    assert np.array_equal(got_codes, want["lat8"])
    assert np.array_equal(np.isnan(got_scale), np.isnan(want["scale"]))
    fin = ~np.isnan(want["scale"])
    assert np.array_equal(got_scale[fin].view(np.uint32), want["scale"][fin].view(np.uint32))
    assert np.isnan(want["scale"][:3]).all() and (want["lat8"][:3] == 0x7F).all()
    assert np.isfinite(want["scale"][3]) and np.isinf(want["scale"][4:6]).all()
    got_rope = kv.rope16()[torch.from_numpy(smap).long()].cpu().numpy().view(np.uint16)
    rnan = np.isnan(src[:, 512:])
    assert np.array_equal(got_rope[~rnan], want["rope16"][~rnan])
    assert ((got_rope[rnan] & 0x7FFF) > 0x7F80).all()
