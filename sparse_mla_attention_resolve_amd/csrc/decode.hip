// a2 + a3 (+ a4, a8): split decode attention over a block table.
//
// Stage 1 (one workgroup per token and split) walks the split's rows in chunks of 32:
// it gathers the chunk's 576-wide rows from the pool into LDS, computes the scores of
// all 64 heads against them with bf16 MFMA (the heads of one token are the M dimension,
// the rows the N dimension), keeps a running max and sum per head (online softmax), and
// accumulates P * V with MFMA, V being the first 512 columns of the same rows. It writes
// the split's normalised output and log-sum-exp. Stage 2 merges a token's splits by LSE
// (IBM Triton paged-attention explainer, section 4 table: "Q-Block" for stacking the
// heads that share a KV row, "Parallel Tiled Softmax" for the split and merge).
//
// The block table is either resolved slots (page size 1, the virtual block table of
// The Virtual Block Table: Reusing Triton MLA for Sparse Attention on Blackwell GPUs,
// "The Breakthrough") or page ids (page size P > 1, the dense paged walk of "The
// Investigation"). fp8 caches are dequantised in the kernel: e4m3 codes convert to
// bf16 exactly, the per-row scale multiplies the latent part of the score and the
// softmax weight that meets the row's values.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int kHeads = 64;
constexpr int kThreads = 256;
constexpr int kRowBytesBf16 = 1152;
constexpr int kLdsRowBf16 = 1168;     // 73 x 16 B: padded so 16 rows hit distinct banks
constexpr int kLdsRowFp8 = 672;       // 42 x 16 B (656-byte packed row + pad)
constexpr int kPStride = 40;          // bf16 per head row of the P tile (80 B)

struct Stage1Args {
  const uint16_t* q;
  int64_t q_tok_stride, q_head_stride;
  smla_kv kv;
  const int32_t* table;
  int64_t table_stride;
  const int32_t* lens;
  int32_t max_len;
  int32_t log2_page;
  float scale_log2;         // softmax scale * log2(e): scores are kept in base 2
  int32_t rows_per_split;
  int32_t S;
  int32_t H;
  float* part_o;            // [T][S][H][512]
  float* part_lse;          // [T][S][H], natural log
};

// Physical slot of position p of token t's table row, or -1 when masked.
__device__ __forceinline__ int64_t slot_of(const Stage1Args& a, int t, int p) {
  const int32_t* row = a.table + (int64_t)t * a.table_stride;
  int64_t s;
  if (a.log2_page == 0) {
    s = row[p];
  } else {
    const int32_t page = row[p >> a.log2_page];
    s = page < 0 ? -1 : ((int64_t)page << a.log2_page) + (p & ((1 << a.log2_page) - 1));
  }
  return (s >= 0 && s < a.kv.num_slots) ? s : -1;
}

__device__ __forceinline__ int token_len(const Stage1Args& a, int t) {
  int n = a.lens[t];
  return n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
}

template <int KV>
struct KvTraits;
template <>
struct KvTraits<SMLA_BF16> {
  static constexpr int kUnits = 72;             // 16-byte units per row
  static constexpr int kLdsRow = kLdsRowBf16;
  static constexpr int kPerThread = (kChunk * kUnits + kThreads - 1) / kThreads;   // 9
  __device__ static const char* unit_src(const smla_kv& kv, int64_t slot, int u) {
    return (const char*)kv.rows + slot * kv.row_stride + u * 16;
  }
};
template <>
struct KvTraits<SMLA_FP8_E4M3> {
  static constexpr int kUnits = 41;             // 32 latent + 8 rope + 1 scale
  static constexpr int kLdsRow = kLdsRowFp8;
  static constexpr int kPerThread = (kChunk * kUnits + kThreads - 1) / kThreads;   // 6
  __device__ static const char* unit_src(const smla_kv& kv, int64_t slot, int u) {
    if (u < 32) return (const char*)kv.lat8 + slot * kv.lat8_stride + u * 16;
    if (u < 40) return (const char*)kv.rope16 + slot * kv.rope16_stride + (u - 32) * 16;
    return (const char*)kv.scale + slot * kv.scale_stride;   // 4 useful bytes of 16 read
  }
};

template <int KV>
__global__ void __launch_bounds__(kThreads, 1) decode_stage1_mfma(Stage1Args a) {
  using Tr = KvTraits<KV>;
  constexpr int kBuf = kChunk * Tr::kLdsRow;
  __shared__ __attribute__((aligned(16))) char kvbuf[2][kBuf];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[kHeads * kPStride];
  __shared__ float xch[2][kHeads];

  const int t = blockIdx.x / a.S;
  const int s = blockIdx.x % a.S;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int hh = w >> 1;      // head half: heads 32hh .. 32hh+31
  const int x = w & 1;        // score phase: row half of the chunk; PV phase: column half

  const int len = token_len(a, t);
  const int r0 = s * a.rows_per_split;
  if (r0 >= len) return;      // inactive split: stage 2 never reads it
  const int r1 = min(r0 + a.rows_per_split, len);
  const int nchunks = (r1 - r0 + kChunk - 1) / kChunk;

  // q fragments (A operand): head hh*32 + 16mt + c, dims 32ks + 8g .. +7
  bf16x8 qf[2][18];
  {
    const uint16_t* qt = a.q + (int64_t)t * a.q_tok_stride;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint16_t* qh = qt + (int64_t)(hh * 32 + mt * 16 + c) * a.q_head_stride;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[mt][ks] = as_bf16x8(*(const uint4*)(qh + ks * 32 + 8 * g));
    }
  }

  // stage the chunk that starts at position p0 into registers
  uint4 stage[Tr::kPerThread];
  auto gather = [&](int p0) {
#pragma unroll
    for (int k = 0; k < Tr::kPerThread; ++k) {
      const int u = tid + kThreads * k;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (u < kChunk * Tr::kUnits) {
        const int row = u / Tr::kUnits, col = u % Tr::kUnits;
        const int p = p0 + row;
        if (p < r1) {
          const int64_t slot = slot_of(a, t, p);
          if (slot >= 0) {
            const char* src = Tr::unit_src(a.kv, slot, col);
            if (KV == SMLA_FP8_E4M3 && col == 40)
              v.x = *(const uint32_t*)src;
            else
              v = *(const uint4*)src;
          }
        }
      }
      stage[k] = v;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < Tr::kPerThread; ++k) {
      const int u = tid + kThreads * k;
      if (u < kChunk * Tr::kUnits) {
        const int row = u / Tr::kUnits, col = u % Tr::kUnits;
        *(uint4*)(kvbuf[buf] + row * Tr::kLdsRow + col * 16) = stage[k];
      }
    }
  };

  f32x4 oacc[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2][4], l_run[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) { m_run[mt][v] = -INFINITY; l_run[mt][v] = 0.f; }

  gather(r0);
  commit(0);
  __syncthreads();

  for (int ci = 0; ci < nchunks; ++ci) {
    const int buf = ci & 1;
    const int p0 = r0 + ci * kChunk;
    if (ci + 1 < nchunks) gather(p0 + kChunk);
    const char* kb = kvbuf[buf];

    // ---- scores: heads hh*32 + 16mt + (4g+v), row x*16 + c of the chunk
    const int myrow = x * 16 + c;
    const char* krow = kb + myrow * Tr::kLdsRow;
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    float rowscale = 1.0f;
    if constexpr (KV == SMLA_BF16) {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const bf16x8 kf = as_bf16x8(*(const uint4*)(krow + (ks * 32 + 8 * g) * 2));
        sacc[0] = mfma16x16x32(qf[0][ks], kf, sacc[0]);
        sacc[1] = mfma16x16x32(qf[1][ks], kf, sacc[1]);
      }
    } else {
      f32x4 racc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint2 codes = *(const uint2*)(krow + ks * 32 + 8 * g);
        const bf16x8 kf = e4m3x8_to_bf16x8(codes.x, codes.y);
        sacc[0] = mfma16x16x32(qf[0][ks], kf, sacc[0]);
        sacc[1] = mfma16x16x32(qf[1][ks], kf, sacc[1]);
      }
#pragma unroll
      for (int ks = 16; ks < 18; ++ks) {
        const bf16x8 kf = as_bf16x8(*(const uint4*)(krow + SMLA_FP8_ROPE_OFFSET + ((ks - 16) * 32 + 8 * g) * 2));
        racc[0] = mfma16x16x32(qf[0][ks], kf, racc[0]);
        racc[1] = mfma16x16x32(qf[1][ks], kf, racc[1]);
      }
      rowscale = *(const float*)(krow + SMLA_FP8_SCALE_OFFSET);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sacc[mt][v] = sacc[mt][v] * rowscale + racc[mt][v];
    }
    const int p = p0 + myrow;
    const bool row_ok = p < r1 && slot_of(a, t, p) >= 0;
    float sv[2][4], mloc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[mt][v] = row_ok ? sacc[mt][v] * a.scale_log2 : -INFINITY;
        mloc[mt][v] = max16(sv[mt][v]);
      }
    if (c == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) xch[x][hh * 32 + mt * 16 + 4 * g + v] = mloc[mt][v];
    }
    __syncthreads();
    float alpha[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = hh * 32 + mt * 16 + 4 * g + v;
        const float mc = fmaxf(mloc[mt][v], xch[x ^ 1][h]);
        const float mn = fmaxf(m_run[mt][v], mc);
        const bool none = mn == -INFINITY;
        alpha[mt][v] = none ? 1.0f : exp2f(m_run[mt][v] - mn);
        const float pv = none ? 0.0f : exp2f(sv[mt][v] - mn);
        l_run[mt][v] = l_run[mt][v] * alpha[mt][v] + sum16(pv);
        m_run[mt][v] = mn;
        pbuf[h * kPStride + myrow] = (uint16_t)f32_to_bf16_rne(pv * rowscale);
      }
    __syncthreads();

    // ---- P * V: heads hh*32 + 16mt + (4g+v), columns x*256 + 16nt + c
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) oacc[mt][nt][v] *= alpha[mt][v];
    bf16x8 pf[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      pf[mt] = as_bf16x8(*(const uint4*)(pbuf + (hh * 32 + mt * 16 + c) * kPStride + 8 * g));
#pragma unroll
    for (int nt = 0; nt < 16; ++nt) {
      const int col = x * 256 + nt * 16 + c;
      bf16x8 vf;
      if constexpr (KV == SMLA_BF16) {
        uint32_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = *(const uint16_t*)(kb + (8 * g + i) * Tr::kLdsRow + col * 2);
        vf = as_bf16x8(make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                  e[6] | (e[7] << 16)));
      } else {
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = *(const uint8_t*)(kb + (8 * g + i) * Tr::kLdsRow + col);
        vf = e4m3x8_to_bf16x8(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                              b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
      }
      oacc[0][nt] = mfma16x16x32(pf[0], vf, oacc[0][nt]);
      oacc[1][nt] = mfma16x16x32(pf[1], vf, oacc[1][nt]);
    }
    if (ci + 1 < nchunks) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- combine the two row halves' sums, normalise, write the split's partials
  if (c == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) xch[x][hh * 32 + mt * 16 + 4 * g + v] = l_run[mt][v];
  }
  __syncthreads();
  const int64_t part = (int64_t)t * a.S + s;
  float* po = a.part_o + part * a.H * kLatent;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hh * 32 + mt * 16 + 4 * g + v;
      const float l = xch[0][h] + xch[1][h];
      const float inv = l > 0.f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) po[h * kLatent + x * 256 + nt * 16 + c] = oacc[mt][nt][v] * inv;
      if (x == 0 && c == 0)
        a.part_lse[part * a.H + h] = l > 0.f ? (m_run[mt][v] + log2f(l)) * kLn2 : -INFINITY;
    }
}

// fp32 q and fp32 cache: a plain VALU path, 16 heads per workgroup, rows in chunks of 16.
__global__ void __launch_bounds__(kThreads) decode_stage1_f32(Stage1Args a) {
  constexpr int kR = 16;
  __shared__ float qs[16][kRow + 4];
  __shared__ float ks[kR][kRow + 4];
  __shared__ float ps[16][kR];
  const int t = blockIdx.x / a.S, s = blockIdx.x % a.S, h0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  const int hl = tid >> 4, n = tid & 15;
  const int len = token_len(a, t);
  const int r0 = s * a.rows_per_split;
  if (r0 >= len) return;
  const int r1 = min(r0 + a.rows_per_split, len);
  const float* qf = (const float*)a.q;
  for (int i = tid; i < 16 * kRow; i += kThreads) {
    const int hh = i / kRow, d = i % kRow;
    qs[hh][d] = (h0 + hh < a.H) ? qf[(int64_t)t * a.q_tok_stride + (int64_t)(h0 + hh) * a.q_head_stride + d] : 0.f;
  }
  float o[32];
  for (int k = 0; k < 32; ++k) o[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int p0 = r0; p0 < r1; p0 += kR) {
    __syncthreads();
    for (int i = tid; i < kR * kRow; i += kThreads) {
      const int rr = i / kRow, d = i % kRow;
      const int p = p0 + rr;
      float v = 0.f;
      if (p < r1) {
        const int64_t slot = slot_of(a, t, p);
        if (slot >= 0) v = *(const float*)((const char*)a.kv.rows + slot * a.kv.row_stride + d * 4);
      }
      ks[rr][d] = v;
    }
    __syncthreads();
    const int p = p0 + n;
    float sc = -INFINITY;
    if (p < r1 && slot_of(a, t, p) >= 0) {
      float acc = 0.f;
      for (int d = 0; d < kRow; ++d) acc = fmaf(qs[hl][d], ks[n][d], acc);
      sc = acc * a.scale_log2;
    }
    const float mn = fmaxf(m_run, max16(sc));
    const bool none = mn == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - mn);
    const float pv = none ? 0.f : exp2f(sc - mn);
    l_run = l_run * alpha + sum16(pv);
    m_run = mn;
    ps[hl][n] = pv;
    __syncthreads();
    for (int k = 0; k < 32; ++k) {
      const int col = n + 16 * k;
      float acc = o[k] * alpha;
      for (int r = 0; r < kR; ++r) acc = fmaf(ps[hl][r], ks[r][col], acc);
      o[k] = acc;
    }
  }
  const int h = h0 + hl;
  if (h >= a.H) return;
  const int64_t part = (int64_t)t * a.S + s;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  for (int k = 0; k < 32; ++k) a.part_o[(part * a.H + h) * kLatent + n + 16 * k] = o[k] * inv;
  if (n == 0) a.part_lse[part * a.H + h] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

struct Stage2Args {
  const int32_t* lens;
  int32_t max_len;
  int32_t rows_per_split;
  int32_t S, H;
  const float* part_o;
  const float* part_lse;
  void* out;
  int64_t out_tok_stride, out_head_stride;
  float* lse;
  int64_t lse_tok_stride;
  int32_t out_f32;
};

// One workgroup per token and 8 heads; thread = (head, 16 consecutive columns).
__global__ void __launch_bounds__(256) decode_stage2(Stage2Args a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 8 + (threadIdx.x >> 5);
  const int c0 = (threadIdx.x & 31) * 16;
  if (h >= a.H) return;
  int len = a.lens[t];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int nact = min(a.S, (len + a.rows_per_split - 1) / a.rows_per_split);
  const int64_t base = (int64_t)t * a.S;
  float mx = -INFINITY;
  for (int s = 0; s < nact; ++s) mx = fmaxf(mx, a.part_lse[(base + s) * a.H + h]);
  float acc[16];
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < nact; ++s) {
      const float l = a.part_lse[(base + s) * a.H + h];
      if (l == -INFINITY) continue;
      const float wgt = expf(l - mx);
      wsum += wgt;
      const float4* src = (const float4*)(a.part_o + ((base + s) * a.H + h) * kLatent + c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = src[i];
        acc[4 * i] += wgt * v.x;
        acc[4 * i + 1] += wgt * v.y;
        acc[4 * i + 2] += wgt * v.z;
        acc[4 * i + 3] += wgt * v.w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  if (a.out_f32) {
    float* o = (float*)a.out + (int64_t)t * a.out_tok_stride + (int64_t)h * a.out_head_stride + c0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4*)(o + 4 * i) = make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv,
                                          acc[4 * i + 3] * inv);
  } else {
    uint16_t* o = (uint16_t*)a.out + (int64_t)t * a.out_tok_stride + (int64_t)h * a.out_head_stride + c0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint4 v;
      v.x = pack_bf16x2(acc[8 * i] * inv, acc[8 * i + 1] * inv);
      v.y = pack_bf16x2(acc[8 * i + 2] * inv, acc[8 * i + 3] * inv);
      v.z = pack_bf16x2(acc[8 * i + 4] * inv, acc[8 * i + 5] * inv);
      v.w = pack_bf16x2(acc[8 * i + 6] * inv, acc[8 * i + 7] * inv);
      *(uint4*)(o + 8 * i) = v;
    }
  }
  if (a.lse && (threadIdx.x & 31) == 0)
    a.lse[(int64_t)t * a.lse_tok_stride + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_decode(const smla_decode_args& d, const DecodePlan& plan, void* ws, hipStream_t stream,
                         int stages) {
  if (d.T == 0) return hipSuccess;
  Stage1Args a;
  a.q = (const uint16_t*)d.q;
  a.q_tok_stride = d.q_tok_stride;
  a.q_head_stride = d.q_head_stride;
  a.kv = d.kv;
  a.table = d.table;
  a.table_stride = d.table_stride;
  a.lens = d.lens;
  a.max_len = plan.max_len;
  int log2_page = 0;
  while ((1 << log2_page) < d.page_size) ++log2_page;
  a.log2_page = log2_page;
  a.scale_log2 = d.scale * kLog2e;
  a.rows_per_split = plan.rows_per_split;
  a.S = plan.S;
  a.H = d.H;
  a.part_o = (float*)ws;
  a.part_lse = (float*)((char*)ws + plan.part_o_bytes);

  if (!(stages & 1)) {
  } else if (d.q_dtype == SMLA_F32) {
    dim3 grid(plan.S * d.T, (d.H + 15) / 16);
    hipLaunchKernelGGL(decode_stage1_f32, grid, dim3(kThreads), 0, stream, a);
  } else if (d.kv.dtype == SMLA_BF16) {
    hipLaunchKernelGGL(decode_stage1_mfma<SMLA_BF16>, dim3(plan.S * d.T), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_stage1_mfma<SMLA_FP8_E4M3>, dim3(plan.S * d.T), dim3(kThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(stages & 2)) return e;

  Stage2Args b;
  b.lens = d.lens;
  b.max_len = plan.max_len;
  b.rows_per_split = plan.rows_per_split;
  b.S = plan.S;
  b.H = d.H;
  b.part_o = a.part_o;
  b.part_lse = a.part_lse;
  b.out = d.out;
  b.out_tok_stride = d.out_tok_stride;
  b.out_head_stride = d.out_head_stride;
  b.lse = d.lse;
  b.lse_tok_stride = d.lse_tok_stride;
  b.out_f32 = d.q_dtype == SMLA_F32;
  hipLaunchKernelGGL(decode_stage2, dim3(d.T, (d.H + 7) / 8), dim3(256), 0, stream, b);
  return hipGetLastError();
}

}  // namespace smla
