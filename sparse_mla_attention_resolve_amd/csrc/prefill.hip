// Grouped sparse prefill. G consecutive queries with H heads fill one 128-row tile
// (G * H = 128); the tile walks its group's union once and each row keeps only the
// entries whose membership bit names its query (vLLM PR 63104, "Overview": 2, 4 or 8
// queries share a 128-head row; "Details": the union is gathered once with a mask per
// query; "Changes": groups are views of token-major q and the last group may be short).
//
// One workgroup of 8 waves per group. Wave w owns tile rows 16w .. 16w+15 (member
// w*16/H, heads (16w) % H ..) for both the scores and the output, so each row's softmax
// stays inside one wave. Union rows arrive in chunks of 32, staged through LDS.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int kPThreads = 512;
constexpr int kTile = 128;
constexpr int kLdsRow = 1168;       // 1152-byte bf16 row + 16 B pad
constexpr int kUnits = 72;
constexpr int kPerThread = (kChunk * kUnits + kPThreads - 1) / kPThreads;   // 5
constexpr int kPS = 40;             // bf16 per tile row of the P buffer

struct PrefillKArgs {
  const uint16_t* q;
  int64_t q_tok_stride, q_head_stride;
  smla_kv kv;
  const uint32_t* enc;
  int64_t enc_stride;
  const int32_t* lens;
  int32_t Q, H, G, max_len;
  float scale_log2;
  uint16_t* out;
  int64_t out_tok_stride, out_head_stride;
  float* lse;
  int64_t lse_tok_stride;
};

__global__ void __launch_bounds__(kPThreads, 1) prefill_kernel(PrefillKArgs a) {
  __shared__ __attribute__((aligned(16))) char kvbuf[2][kChunk * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[kTile * kPS];
  __shared__ uint32_t mbits[2][kChunk];

  const int grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int member = (16 * w) / a.H;
  const int head0 = (16 * w) % a.H;
  const int qi = grp * a.G + member;
  const bool live = qi < a.Q;
  int n = a.lens[grp];
  n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
  const uint32_t* erow = a.enc + (int64_t)grp * a.enc_stride;

  // A operand: tile row 16w + c = (member, head0 + c), dims 32ks + 8g .. +7
  bf16x8 qf[18];
  {
    const int qsrc = live ? qi : a.Q - 1;     // a short last group repeats its last query
    const uint16_t* qh = a.q + (int64_t)qsrc * a.q_tok_stride + (int64_t)(head0 + c) * a.q_head_stride;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = as_bf16x8(*(const uint4*)(qh + ks * 32 + 8 * g));
  }

  uint4 stage[kPerThread];
  uint32_t stage_bits = 0;
  auto gather = [&](int p0) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int u = tid + kPThreads * k;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (u < kChunk * kUnits) {
        const int row = u / kUnits, col = u % kUnits;
        const int p = p0 + row;
        if (p < n) {
          const uint32_t row_id = erow[p] & ((1u << SMLA_UNION_ROW_BITS) - 1u);
          if (row_id < a.kv.num_slots)
            v = *(const uint4*)((const char*)a.kv.rows + (int64_t)row_id * a.kv.row_stride + col * 16);
        }
      }
      stage[k] = v;
    }
    if (tid < kChunk) {
      const int p = p0 + tid;
      uint32_t bits = 0;
      if (p < n) {
        const uint32_t e = erow[p];
        if ((e & ((1u << SMLA_UNION_ROW_BITS) - 1u)) < a.kv.num_slots) bits = e >> SMLA_UNION_ROW_BITS;
      }
      stage_bits = bits;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int u = tid + kPThreads * k;
      if (u < kChunk * kUnits) {
        const int row = u / kUnits, col = u % kUnits;
        *(uint4*)(kvbuf[buf] + row * kLdsRow + col * 16) = stage[k];
      }
    }
    if (tid < kChunk) mbits[buf][tid] = stage_bits;
  };

  f32x4 oacc[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_run[v] = -INFINITY; l_run[v] = 0.f; }

  const int nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks > 0) {
    gather(0);
    commit(0);
  }
  __syncthreads();

  for (int ci = 0; ci < nchunks; ++ci) {
    const int buf = ci & 1;
    if (ci + 1 < nchunks) gather((ci + 1) * kChunk);
    const char* kb = kvbuf[buf];

    // scores for tile rows 16w + 4g + v against chunk rows 16j + c (j = 0, 1)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 kf = as_bf16x8(*(const uint4*)(kb + (16 * j + c) * kLdsRow + (ks * 32 + 8 * g) * 2));
        sacc[j] = mfma16x16x32(qf[ks], kf, sacc[j]);
      }
    }
    float sv[2][4];
    float mloc[4], alpha[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = (mbits[buf][16 * j + c] >> member) & 1u;
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[j][v] = ok ? sacc[j][v] * a.scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mloc[v] = max16(fmaxf(sv[0][v], sv[1][v]));
      const float mn = fmaxf(m_run[v], mloc[v]);
      const bool none = mn == -INFINITY;
      alpha[v] = none ? 1.f : exp2f(m_run[v] - mn);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float pv = none ? 0.f : exp2f(sv[j][v] - mn);
        psum += pv;
        pbuf[(16 * w + 4 * g + v) * kPS + 16 * j + c] = (uint16_t)f32_to_bf16_rne(pv);
      }
      l_run[v] = l_run[v] * alpha[v] + sum16(psum);
      m_run[v] = mn;
    }
    __syncthreads();

    const bf16x8 pf = as_bf16x8(*(const uint4*)(pbuf + (16 * w + c) * kPS + 8 * g));
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) oacc[nt][v] *= alpha[v];
      const int col = nt * 16 + c;
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = *(const uint16_t*)(kb + (8 * g + i) * kLdsRow + col * 2);
      const bf16x8 vf = as_bf16x8(make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                             e[6] | (e[7] << 16)));
      oacc[nt] = mfma16x16x32(pf, vf, oacc[nt]);
    }
    if (ci + 1 < nchunks) commit(buf ^ 1);
    __syncthreads();
  }

  if (!live) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = head0 + 4 * g + v;
    const float inv = l_run[v] > 0.f ? 1.0f / l_run[v] : 0.f;
    uint16_t* o = a.out + (int64_t)qi * a.out_tok_stride + (int64_t)h * a.out_head_stride;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) o[nt * 16 + c] = (uint16_t)f32_to_bf16_rne(oacc[nt][v] * inv);
    if (a.lse && c == 0)
      a.lse[(int64_t)qi * a.lse_tok_stride + h] = l_run[v] > 0.f ? (m_run[v] + log2f(l_run[v])) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill(const smla_prefill_args& d, hipStream_t stream) {
  if (d.Q == 0) return hipSuccess;
  if (d.H == 64) return launch_union_decode(d, stream);
  PrefillKArgs a;
  a.q = (const uint16_t*)d.q;
  a.q_tok_stride = d.q_tok_stride;
  a.q_head_stride = d.q_head_stride;
  a.kv = d.kv;
  a.enc = d.enc;
  a.enc_stride = d.enc_stride;
  a.lens = d.lens;
  a.Q = d.Q;
  a.H = d.H;
  a.G = d.G;
  a.max_len = d.enc_width;
  a.scale_log2 = d.scale * kLog2e;
  a.out = (uint16_t*)d.out;
  a.out_tok_stride = d.out_tok_stride;
  a.out_head_stride = d.out_head_stride;
  a.lse = d.lse;
  a.lse_tok_stride = d.lse_tok_stride;
  const int groups = (d.Q + d.G - 1) / d.G;
  hipLaunchKernelGGL(prefill_kernel, dim3(groups), dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
