"""Number formats used by the cache, written from their definitions.

Test infrastructure only (see the package header).

bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent, 7 fraction bits).

fp8 e4m3 ("E4M3FN" in the OCP 8-bit floating point specification): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
m/8 * 2^-6; there are no infinities, and S.1111.111 is NaN, so the largest finite
magnitude is 1.75 * 2^8 = 448. The fp8 KV cache of the pages is this format (The
Assertion That Changed Everything, "Why This Message Was Written": the
fp8_e4m3 kv-cache dtype).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 to each float32 value, ties to the even pattern; returns uint16 bits.

    Written as the definition: the two bf16 neighbours of x are x with its low 16 bits
    cleared (toward zero) and the next pattern away from zero; take the closer, and on a
    tie the one whose last kept bit is 0. NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    toward = (u & np.uint32(0xFFFF0000)).astype(np.uint64)
    away = toward + 0x10000
    v = x.astype(np.float64)
    vt = (toward.astype(np.uint32)).view(np.float32).astype(np.float64)
    va = (away.astype(np.uint32)).view(np.float32).astype(np.float64)
    # stepping past the largest finite pattern reaches the infinity pattern; for the
    # rounding decision it stands for 2^128, the next value of an unbounded exponent, so
    # that values beyond max + half an ulp round to infinity as IEEE rounding requires
    va = np.where(np.isinf(va), np.copysign(2.0 ** 128, va), va)
    dt = np.abs(v - vt)
    da = np.abs(va - v)
    pick_away = (da < dt) | ((da == dt) & (((toward >> 16) & 1) == 1))
    out = np.where(pick_away, away, toward) >> 16
    out = out.astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


# the 127 finite non-negative codes and their values, in increasing order
_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round each value to e4m3: the nearest finite e4m3 value, ties to the even code,
    magnitudes beyond 448 saturated to 448; the sign is kept (including -0). NaN in -> NaN
    code 0x7F."""
    v = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = _POS_VALUES[hi] == a
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    code[np.isnan(v)] = 0x7F
    return code
