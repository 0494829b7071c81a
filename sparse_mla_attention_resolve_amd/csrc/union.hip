// Per-group top-k union with membership bits (vLLM PR 63104, "Tests" for the edge
// cases, "Changes" for unions of consecutive queries whose rows keep a bit per member,
// "Details" for gathering the union once per 128-row tile).
//
// One workgroup per group. Small pools use a map of the pool's rows in LDS (below); otherwise
// every listed (row, member) pair becomes the key
// row * 8 + member; padding, negative rows and rows past the pool become 0xffffffff.
// The keys are sorted in LDS (bitonic network), equal rows end up adjacent, each run of
// one row is folded into a single entry whose member bits are OR-ed, and a block-wide
// prefix count of run heads gives every entry its place in the ascending output.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int kUnionThreads = 1024;
constexpr int kMaxKeys = 16384;
constexpr uint32_t kEmpty = 0xffffffffu;

__global__ void __launch_bounds__(kUnionThreads) union_kernel(
    const int32_t* __restrict__ slots, int64_t slots_stride, const int32_t* __restrict__ valid,
    int32_t Q, int32_t W, int32_t G, int32_t num_keys_pow2, int64_t num_slots,
    uint32_t* __restrict__ enc, int64_t enc_stride, int32_t* __restrict__ lens) {
  __shared__ uint32_t keys[kMaxKeys];
  __shared__ int32_t wave_tot[kUnionThreads / 64];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = num_keys_pow2;

  for (int i = tid; i < n; i += kUnionThreads) {
    uint32_t key = kEmpty;
    const int m = i / W, j = i - m * W;
    const int q = g * G + m;
    if (m < G && q < Q) {
      const int cnt = valid ? valid[q] : W;
      if (j < cnt) {
        const int32_t r = slots[(int64_t)q * slots_stride + j];
        if (r >= 0 && r < num_slots) key = ((uint32_t)r << 3) | (uint32_t)m;
      }
    }
    keys[i] = key;
  }
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= n; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int pi = tid; pi < (n >> 1); pi += kUnionThreads) {
        const int i = 2 * jj * (pi / jj) + (pi % jj);
        const int l = i + jj;
        const uint32_t a = keys[i], b = keys[l];
        const bool up = (i & k) == 0;
        if ((a > b) == up) { keys[i] = b; keys[l] = a; }
      }
      __syncthreads();
    }
  }

  // each thread owns a contiguous span of the sorted keys
  const int per = (n + kUnionThreads - 1) / kUnionThreads;
  const int b0 = tid * per, b1 = min(b0 + per, n);
  int heads = 0;
  for (int i = b0; i < b1; ++i) {
    const uint32_t key = keys[i];
    if (key != kEmpty && (i == 0 || (keys[i - 1] >> 3) != (key >> 3))) ++heads;
  }
  // block-wide exclusive scan of the head counts
  const int lane = tid & 63, wv = tid >> 6;
  int incl = heads;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int k2 = 0; k2 < wv; ++k2) before += wave_tot[k2];
  int pos = before + incl - heads;
  uint32_t* out = enc + (int64_t)g * enc_stride;
  for (int i = b0; i < b1; ++i) {
    const uint32_t key = keys[i];
    if (key == kEmpty || (i > 0 && (keys[i - 1] >> 3) == (key >> 3))) continue;
    const uint32_t row = key >> 3;
    uint32_t mask = 0;
    for (int k2 = i; k2 < n && keys[k2] != kEmpty && (keys[k2] >> 3) == row; ++k2) mask |= 1u << (keys[k2] & 7u);
    out[pos++] = row | (mask << SMLA_UNION_ROW_BITS);
  }
  if (tid == kUnionThreads - 1) lens[g] = pos;
}

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
  int n = 1;
  while (n < G * W) n <<= 1;
  hipLaunchKernelGGL(union_kernel, dim3(groups), dim3(kUnionThreads), 0, stream, slots, slots_stride,
                     valid, Q, W, G, n, num_slots, enc, enc_stride, lens);
  return hipGetLastError();
}

}  // namespace smla
