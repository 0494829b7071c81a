// Per-group top-k union with membership bits (vLLM PR 63104, "Tests" for the edge
// cases, "Changes" for unions of consecutive queries whose rows keep a bit per member,
// "Details" for gathering the union once per 128-row tile).
//
// One workgroup per group, two builders with the same result (the ascending union, each row
// once with the OR of its members' bits):
//   - pools of up to kMapSlots rows: a map of one byte per pool row in LDS;
//   - larger pools: every listed (row, member) pair becomes the key row * 8 + member (padding,
//     negative rows and rows past the pool become 0xffffffff), the keys are sorted by a
//     bitonic network held in registers, each run of one row is folded into a single entry,
//     and a block-wide prefix count of run heads gives every entry its place.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int kUnionThreads = 1024;
constexpr uint32_t kEmpty = 0xffffffffu;

// Pools of at most kMapSlots rows: the group marks its members in a map of one byte per
// pool row in LDS (bit m of row r's byte = member m lists r; an atomic OR per listed entry),
// then walks the map in ascending row order: thread i owns rows [i * per, (i + 1) * per), and
// a block-wide prefix count of the marked rows gives every entry its place. No sort, and the
// result is the same ascending union with the same bits.
constexpr int kMapSlots = 49152;

__global__ void __launch_bounds__(kUnionThreads) union_map_kernel(
    const int32_t* __restrict__ slots, int64_t slots_stride, const int32_t* __restrict__ valid,
    int32_t Q, int32_t W, int32_t G, int32_t num_slots, int32_t per,
    uint32_t* __restrict__ enc, int64_t enc_stride, int32_t* __restrict__ lens) {
  extern __shared__ uint32_t map[];                      // (num_slots + 3) / 4 words
  __shared__ int32_t wave_tot[kUnionThreads / 64];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int nwords = (num_slots + 3) >> 2;
  for (int i = tid; i < nwords; i += kUnionThreads) map[i] = 0u;
  __syncthreads();
  for (int m = 0; m < G; ++m) {
    const int q = g * G + m;
    if (q >= Q) break;
    const int cnt = valid ? min(max(valid[q], 0), W) : W;
    const int32_t* row = slots + (int64_t)q * slots_stride;
    for (int j = tid; j < cnt; j += kUnionThreads) {
      const int32_t r = row[j];
      if (r >= 0 && r < num_slots) atomicOr(&map[r >> 2], (1u << m) << (8 * (r & 3)));
    }
  }
  __syncthreads();
  // this thread's rows: per is a multiple of 4, so they are whole words
  const int r0 = tid * per, r1 = min(r0 + per, num_slots);
  int heads = 0;
  for (int r = r0; r < r1; r += 4) {
    const uint32_t v = map[r >> 2];
    heads += ((v & 0xffu) != 0) + ((v & 0xff00u) != 0) + ((v & 0xff0000u) != 0) + ((v >> 24) != 0);
  }
  const int lane = tid & 63, wv = tid >> 6;
  int incl = heads;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int k2 = 0; k2 < kUnionThreads / 64; ++k2) {
    before += k2 < wv ? wave_tot[k2] : 0;
    total += wave_tot[k2];
  }
  int pos = before + incl - heads;
  uint32_t* out = enc + (int64_t)g * enc_stride;
  for (int r = r0; r < r1; r += 4) {
    const uint32_t v = map[r >> 2];
    if (v == 0u) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t mask = (v >> (8 * b)) & 0xffu;
      if (mask != 0u) out[pos++] = (uint32_t)(r + b) | (mask << SMLA_UNION_ROW_BITS);
    }
  }
  if (tid == 0) lens[g] = total;
}

// Pools too large for the row map: the group's keys (row << 3 | member, empty = 0xffffffff)
// are sorted by a bitonic network whose data stays in registers, unrolled at compile time.
// Thread t holds keys t*K .. t*K + K - 1 of the n = P * K (a power of two); a compare-exchange
// of stride j pairs key p with key p ^ j, which is
//   - in the same thread for j < K (register pairs),
//   - in lane t ^ (j / K) of the same wave for K <= j < 64 K (a DPP or swizzle lane move,
//     a permute for the 32-lane stride),
//   - in another wave for j >= 64 K (through LDS, between barriers; the last few strides only).
// Whether a pair sorts up or down and which side keeps the smaller key depend only on the
// stage, the stride and the thread, so each step's choice is made once per thread.
// Then, as in the other builder, each run of one row is folded into one entry whose member
// bits are OR-ed, and a block-wide count of run heads places the entries in ascending order.
template <int TM>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (TM == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
  else if constexpr (TM == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false);  // 2,3,0,1
  else if constexpr (TM < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (TM << 10) | 0x1f);  // xor within 32
  else return (uint32_t)__shfl_xor((int)v, TM, 64);
}

__device__ __forceinline__ void cx(uint32_t& a, uint32_t& b, bool up) {
  const uint32_t lo = a < b ? a : b, hi = a < b ? b : a;
  a = up ? lo : hi;
  b = up ? hi : lo;
}

// one step (stage size S, stride J) of the network over the thread's K keys
template <int P, int K, int S, int J>
__device__ __forceinline__ void sort_step(uint32_t (&v)[K], uint32_t* keys, int t) {
  if constexpr (J < K) {
#pragma unroll
    for (int i = 0; i < K; ++i)
      if ((i & J) == 0) cx(v[i], v[i | J], S < K ? ((i & S) == 0) : (((t * K) & S) == 0));
  } else if constexpr (J < 64 * K) {
    const bool up = ((t * K) & S) == 0, lower = (t & (J / K)) == 0;
    const bool keep_lo = up == lower;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t pv = lane_xor<J / K>(v[i]);
      v[i] = keep_lo ? (v[i] < pv ? v[i] : pv) : (v[i] < pv ? pv : v[i]);
    }
  } else {
    const bool up = ((t * K) & S) == 0, lower = ((t * K) & J) == 0;
    const bool keep_lo = up == lower;
    __syncthreads();                                       // the previous exchange is read
#pragma unroll
    for (int i = 0; i < K; ++i) keys[t * K + i] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t pv = keys[(t * K + i) ^ J];
      v[i] = keep_lo ? (v[i] < pv ? v[i] : pv) : (v[i] < pv ? pv : v[i]);
    }
  }
}

template <int P, int K, int S, int J>
__device__ __forceinline__ void sort_stage(uint32_t (&v)[K], uint32_t* keys, int t) {
  sort_step<P, K, S, J>(v, keys, t);
  if constexpr (J > 1) sort_stage<P, K, S, J / 2>(v, keys, t);
}

template <int P, int K, int S>
__device__ __forceinline__ void sort_all(uint32_t (&v)[K], uint32_t* keys, int t) {
  sort_stage<P, K, S, S / 2>(v, keys, t);
  if constexpr (S < P * K) sort_all<P, K, S * 2>(v, keys, t);
}

template <int P, int K>
__global__ void __launch_bounds__(P) union_sort_kernel(
    const int32_t* __restrict__ slots, int64_t slots_stride, const int32_t* __restrict__ valid,
    int32_t Q, int32_t W, int32_t G, int64_t num_slots,
    uint32_t* __restrict__ enc, int64_t enc_stride, int32_t* __restrict__ lens) {
  constexpr int n = P * K;
  __shared__ uint32_t keys[n];
  __shared__ int32_t wave_tot[P / 64];
  const int g = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t v[K];
  // the thread's keys before the sort: entries t, t + P, t + 2P, ... of the members' lists laid
  // end to end (any assignment sorts the same; this one makes each load instruction contiguous)
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int e = i * P + t;
    const int m = e / W, j = e - m * W;
    uint32_t key = kEmpty;
    const int q = g * G + m;
    if (m < G && q < Q) {
      const int cnt = valid ? min(max(valid[q], 0), W) : W;
      if (j < cnt) {
        const int32_t r = slots[(int64_t)q * slots_stride + j];
        if (r >= 0 && r < num_slots) key = ((uint32_t)r << 3) | (uint32_t)m;
      }
    }
    v[i] = key;
  }
  sort_all<P, K, 2>(v, keys, t);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i) keys[t * K + i] = v[i];
  __syncthreads();
  // run heads in this thread's span, then a block-wide exclusive count of them
  int heads = 0;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int p = t * K + i;
    if (v[i] != kEmpty && (p == 0 || (keys[p - 1] >> 3) != (v[i] >> 3))) ++heads;
  }
  int incl = heads;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int k2 = 0; k2 < P / 64; ++k2) {
    before += k2 < wv ? wave_tot[k2] : 0;
    total += wave_tot[k2];
  }
  int pos = before + incl - heads;
  uint32_t* out = enc + (int64_t)g * enc_stride;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int p = t * K + i;
    const uint32_t key = v[i];
    if (key == kEmpty || (p > 0 && (keys[p - 1] >> 3) == (key >> 3))) continue;
    const uint32_t row = key >> 3;
    uint32_t mask = 0;
    for (int k2 = p; k2 < n && keys[k2] != kEmpty && (keys[k2] >> 3) == row; ++k2) mask |= 1u << (keys[k2] & 7u);
    out[pos++] = row | (mask << SMLA_UNION_ROW_BITS);
  }
  if (t == 0) lens[g] = total;
}

}  // namespace

hipError_t launch_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                        int32_t Q, int32_t W, int32_t G, int64_t num_slots, uint32_t* enc,
                        int64_t enc_stride, int32_t* lens, hipStream_t stream) {
  if (Q == 0) return hipSuccess;
  const int groups = (Q + G - 1) / G;
  if (num_slots <= kMapSlots) {
    const int per = ((int)((num_slots + kUnionThreads - 1) / kUnionThreads) + 3) / 4 * 4;
    const size_t lds = (size_t)((num_slots + 3) / 4) * 4;
    hipLaunchKernelGGL(union_map_kernel, dim3(groups), dim3(kUnionThreads), lds, stream, slots, slots_stride, valid,
                       Q, W, G, (int32_t)num_slots, per, enc, enc_stride, lens);
    return hipGetLastError();
  }
  int n = 256;
  while (n < G * W) n <<= 1;
#define SMLA_UNION_SORT(P, K)                                                                                        \
  hipLaunchKernelGGL((union_sort_kernel<P, K>), dim3(groups), dim3(P), 0, stream, slots, slots_stride, valid, Q, W, G, \
                     num_slots, enc, enc_stride, lens)
  switch (n) {
    case 256: SMLA_UNION_SORT(256, 1); break;
    case 512: SMLA_UNION_SORT(256, 2); break;
    case 1024: SMLA_UNION_SORT(256, 4); break;
    case 2048: SMLA_UNION_SORT(256, 8); break;
    case 4096: SMLA_UNION_SORT(256, 16); break;
    case 8192: SMLA_UNION_SORT(512, 16); break;
    default: SMLA_UNION_SORT(1024, 16); break;    // 16384, the largest G * W the ABI accepts
  }
#undef SMLA_UNION_SORT
  return hipGetLastError();
}

}  // namespace smla
