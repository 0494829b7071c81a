// Device-side helpers shared by the libsmla kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/smla.h"

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = SMLA_LATENT;
constexpr int kRope = SMLA_ROPE;
constexpr int kRow = SMLA_ROW;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Nearest bf16, ties to even; NaN stays NaN; overflow rounds to infinity.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// v_mfma_f32_16x16x32_bf16. With lane = 16*g + c:
//   A operand: A[c][8g .. 8g+7]   (row c of the 16x32 left matrix)
//   B operand: B[8g .. 8g+7][c]   (column c of the 32x16 right matrix)
//   C/D:       D[4g .. 4g+3][c]
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of `w`, by `hi`) to two bf16 values, exact: every
// e4m3 value is a bf16 value, and the scale operand is 1.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight e4m3 codes (little-endian in two words) to eight bf16 values.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint4 v;
  v.x = e4m3x2_to_bf16x2(w0, false);
  v.y = e4m3x2_to_bf16x2(w0, true);
  v.z = e4m3x2_to_bf16x2(w1, false);
  v.w = e4m3x2_to_bf16x2(w1, true);
  return as_bf16x8(v);
}

// Reductions over the 16 lanes that share lane / 16 (one column group of an MFMA tile),
// with DPP lane moves: swap neighbours, swap pairs, mirror within 8, mirror within 16.
// After the four steps every lane of the group holds the group's result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadSwap1 = 0xb1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4e;    // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<kDppQuadSwap1>(v);
  v += dpp<kDppQuadSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

// e4m3 code of a float32 value: nearest, ties to even, magnitudes past 448 saturated
// to 448, sign kept; NaN -> 0x7f. Integer and exact power-of-two steps only.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  if (a != a) return 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                            // below 2^-6: subnormal step 2^-9
    float n = __builtin_rintf(a * 512.0f);       // 0 .. 8, ties to even
    return sign | (uint32_t)n;                   // 8 is the smallest normal, code 0x08
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6 .. 8
  float n = __builtin_rintf(ldexpf(a, 3 - e));              // 8 .. 16, ties to even
  uint32_t r = (uint32_t)n;
  if (r == 16u) { r = 8u; e += 1; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | (r - 8u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no LDS): shifts by 1,
// 2, 4 and 8 lanes inside each row of 16, then the last lane of row 0 added to rows 1 and 3,
// and the last lane of row 1 (by then the sum of rows 0 and 1) added to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x = dpp_add<0x111, 0xf>(x);                          // row_shr:1
  x = dpp_add<0x112, 0xf>(x);                          // row_shr:2
  x = dpp_add<0x114, 0xf>(x);                          // row_shr:4
  x = dpp_add<0x118, 0xf>(x);                          // row_shr:8
  x = dpp_add<0x142, 0xa>(x);                          // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xc>(x);                          // row_bcast:31 into rows 2, 3
  return x;
}

}  // namespace smla
