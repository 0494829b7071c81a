// Per-group top-k union with membership bits (vLLM PR 63104, "Tests" for the edge
// cases, "Changes" for unions of consecutive queries whose rows keep a bit per member,
// "Details" for gathering the union once per 128-row tile).
//
// One workgroup per group. Every listed (row, member) pair becomes the key
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

}  // namespace

hipError_t launch_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                        int32_t Q, int32_t W, int32_t G, int64_t num_slots, uint32_t* enc,
                        int64_t enc_stride, int32_t* lens, hipStream_t stream) {
  if (Q == 0) return hipSuccess;
  int n = 1;
  while (n < G * W) n <<= 1;
  const int groups = (Q + G - 1) / G;
  hipLaunchKernelGGL(union_kernel, dim3(groups), dim3(kUnionThreads), 0, stream, slots, slots_stride,
                     valid, Q, W, G, n, num_slots, enc, enc_stride, lens);
  return hipGetLastError();
}

}  // namespace smla
