// Cache write, bf16 / fp32 / fp8 e4m3 with a per-token scale. The Assertion That
// Changed Everything, "The Message" (the write into the pool that precedes decode
// attention, and the fp8 cache the Triton path refused) and "Why This Message Was
// Written" (the fp8_e4m3 cache dtype).
#include <type_traits>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

// One 64-lane wave per token row. Lane l owns latent columns 8l .. 8l+7 and rotary
// column l.
__global__ void __launch_bounds__(64) kv_write_kernel(
    const void* __restrict__ src, int32_t src_dtype, int64_t src_stride,
    const int32_t* __restrict__ slot_mapping, int32_t T, smla_kv dst) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || slot >= dst.num_slots) return;

  float lat[8];
  float rope;
  if (src_dtype == SMLA_F32) {
    const float* s = (const float*)src + (int64_t)t * src_stride;
    float4 a = *(const float4*)(s + 8 * lane);
    float4 b = *(const float4*)(s + 8 * lane + 4);
    lat[0] = a.x; lat[1] = a.y; lat[2] = a.z; lat[3] = a.w;
    lat[4] = b.x; lat[5] = b.y; lat[6] = b.z; lat[7] = b.w;
    rope = s[kLatent + lane];
  } else {
    const uint16_t* s = (const uint16_t*)src + (int64_t)t * src_stride;
    uint4 v = *(const uint4*)(s + 8 * lane);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    for (int i = 0; i < 4; ++i) {
      lat[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      lat[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    rope = bf16_to_f32(s[kLatent + lane]);
  }

  if (dst.dtype == SMLA_F32) {
    float* d = (float*)((char*)dst.rows + (int64_t)slot * dst.row_stride);
    *(float4*)(d + 8 * lane) = make_float4(lat[0], lat[1], lat[2], lat[3]);
    *(float4*)(d + 8 * lane + 4) = make_float4(lat[4], lat[5], lat[6], lat[7]);
    d[kLatent + lane] = rope;
  } else if (dst.dtype == SMLA_BF16) {
    uint16_t* d = (uint16_t*)((char*)dst.rows + (int64_t)slot * dst.row_stride);
    uint4 v;
    v.x = pack_bf16x2(lat[0], lat[1]);
    v.y = pack_bf16x2(lat[2], lat[3]);
    v.z = pack_bf16x2(lat[4], lat[5]);
    v.w = pack_bf16x2(lat[6], lat[7]);
    *(uint4*)(d + 8 * lane) = v;
    d[kLatent + lane] = (uint16_t)f32_to_bf16_rne(rope);
  } else {
    float amax = 0.0f;
    bool nan_in = false;
    for (int i = 0; i < 8; ++i) {
      amax = fmaxf(amax, fabsf(lat[i]));
      nan_in |= lat[i] != lat[i];
    }
    // the row's maximum: a max-scan over the wave with DPP lane moves (row shifts by 1, 2, 4, 8,
    // then rows 0 and 2 into 1 and 3, then row 1 into 2 and 3), lane 63's value in every lane
    // (lanes shifted in from outside a row contribute +0, and every amax is >= +0)
    auto dmax = [](float x, auto ctrl, auto rows) {
      return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                                  decltype(rows)::value, 0xf, false)));
    };
    amax = dmax(amax, std::integral_constant<int, 0x111>(), std::integral_constant<int, 0xf>());
    amax = dmax(amax, std::integral_constant<int, 0x112>(), std::integral_constant<int, 0xf>());
    amax = dmax(amax, std::integral_constant<int, 0x114>(), std::integral_constant<int, 0xf>());
    amax = dmax(amax, std::integral_constant<int, 0x118>(), std::integral_constant<int, 0xf>());
    amax = dmax(amax, std::integral_constant<int, 0x142>(), std::integral_constant<int, 0xa>());
    amax = dmax(amax, std::integral_constant<int, 0x143>(), std::integral_constant<int, 0xc>());
    amax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(amax), 63));
    // fmaxf passes over a NaN; the maximum of a row that holds one is NaN, so its scale is
    // NaN and every latent code of the row is the NaN code
    if (__builtin_amdgcn_ballot_w64(nan_in) != 0) amax = __builtin_nanf("");
    const float scale = amax / 448.0f;              // IEEE division, rounded to nearest
    uint32_t lo = 0, hi = 0;
    if (scale != 0.0f) {
      float qv[8];
      bool nan = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qv[i] = lat[i] / scale;                     // IEEE division, rounded to nearest
        nan |= qv[i] != qv[i];
      }
      if (!nan) {
        // v_cvt_pk_fp8_f32 (ties to even) gives the reference encoder's code for every fp32
        // |x| <= 448, signed zeros and subnormals included (checked on all 2^31.1 such bit
        // patterns); a quotient can pass 448 by rounding, where both give 448, so clamp first
        auto c = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(c(qv[0]), c(qv[1]), 0u, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(c(qv[2]), c(qv[3]), lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(c(qv[4]), c(qv[5]), 0u, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(c(qv[6]), c(qv[7]), hi, true);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3_rne_sat(qv[i]) << (8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3_rne_sat(qv[4 + i]) << (8 * i);
      }
    }
    uint8_t* l8 = (uint8_t*)dst.lat8 + (int64_t)slot * dst.lat8_stride;
    *(uint2*)(l8 + 8 * lane) = make_uint2(lo, hi);
    uint16_t* r16 = (uint16_t*)((char*)dst.rope16 + (int64_t)slot * dst.rope16_stride);
    r16[lane] = (uint16_t)f32_to_bf16_rne(rope);
    if (lane == 0) *(float*)((char*)dst.scale + (int64_t)slot * dst.scale_stride) = scale;
  }
}

hipError_t launch_kv_write(const void* src, int32_t src_dtype, int64_t src_stride,
                           const int32_t* slot_mapping, int32_t T, const smla_kv& dst,
                           hipStream_t stream) {
  hipLaunchKernelGGL(kv_write_kernel, dim3(T), dim3(64), 0, stream, src, src_dtype, src_stride,
                     slot_mapping, T, dst);
  return hipGetLastError();
}

}  // namespace smla
