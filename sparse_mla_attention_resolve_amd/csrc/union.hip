// Per-group top-k union with membership bits (vLLM PR 63104, "Tests" for the edge
// cases, "Changes" for unions of consecutive queries whose rows keep a bit per member,
// "Details" for gathering the union once per 128-row tile).
//
// Two builders with the same result (the ascending union, each row once with the OR of its
// members' bits):
//   - pools of up to kBitmapSlots (2^20) rows, when the map fits LDS: a bit per pool row in LDS
//     (a window of 2^18 rows at a time when a group lists more than 8,192 entries), counted per
//     block to place each row; persistent workgroups build one group after another;
//   - larger pools, one workgroup per group: every listed (row, member) pair becomes the key
//     row * 8 + member (padding, negative rows and rows past the pool become 0xffffffff), the
//     keys are sorted by a bitonic network held in registers, each run of one row is folded
//     into a single entry, and a block-wide prefix count of run heads gives every entry its
//     place.
#include "smla_device.h"
#include "smla_internal.h"

#include <algorithm>
#include <atomic>

namespace smla {

namespace {

constexpr uint32_t kEmpty = 0xffffffffu;

// e / W for 0 <= e < 2^15 and W >= 1, with rw = 1 / W in fp32: the product is within 2^-8 of
// the true quotient, so its truncation is off by at most one, which one step corrects.
__device__ __forceinline__ int div_w(int e, int W, float rw) {
  int m = (int)((float)e * rw);
  m -= m * W > e ? 1 : 0;
  m += (m + 1) * W <= e ? 1 : 0;
  return m;
}

// Workgroup barrier that waits for this wave's LDS operations only: global loads issued ahead
// (the next group's list entries) and the output stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix of x over the P threads of the workgroup (in thread order); `tot` receives
// the sum. wave_tot holds P / 64 words; it is free again after the caller's next barrier.
template <int P>
__device__ __forceinline__ int block_exclusive_sum(int x, int32_t* wave_tot, int& tot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_inclusive_sum(x);
  if (lane == 63) wave_tot[wv] = incl;
  lds_barrier();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int k = 0; k < P / 64; ++k) {
    before += k < wv ? wave_tot[k] : 0;
    tot += wave_tot[k];
  }
  return before + incl - x;
}

// Pools of at most kBitmapSlots rows: a bit per pool row in LDS, in blocks of 128 rows (four
// words), one window of the pool at a time (the whole pool; windows of 2^18 rows for lists of
// more than 8,192 entries, whose map must leave room for their other LDS). The group's listed
// rows set their bits (an atomic OR each). Each wave counts the set bits of a contiguous range
// of blocks, 64 blocks at a time (one 16-byte read per lane, so a wave's reads cover every bank
// once) with a prefix inside the wave, and one block-wide sum of the waves' totals turns the
// counts into the number of union rows before each block. A row's place in the ascending union
// is then its block's count plus the set bits before it in the block (one 16-byte read). Each
// listed entry ORs its member's bit into its place's byte, the union's rows are written over
// the bit map in place order, and one coalesced pass writes the entries; a window's union rows
// follow the previous windows'. Cost per group: the map's size (cleared and counted once per
// window) plus a few LDS reads per listed entry; no sort.
// A workgroup builds groups blockIdx.x, + gridDim.x, ... (as many workgroups as fit the compute
// units at once): the next group's list entries are loaded while the current one is built.
constexpr int kBitmapSlots = 1 << 20;
constexpr int kBitmapThreads = 1024;

template <int K>
__global__ void __launch_bounds__(kBitmapThreads) union_bitmap_kernel(
    const int32_t* __restrict__ slots, int64_t slots_stride, const int32_t* __restrict__ valid,
    int32_t Q, int32_t W, int32_t G, int32_t num_slots, int32_t groups,
    uint32_t* __restrict__ enc, int64_t enc_stride, int32_t* __restrict__ lens) {
  constexpr int P = kBitmapThreads, kWaves = P / 64;
  extern __shared__ uint32_t lds[];
  __shared__ int32_t wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = G * W;                                 // list entries of a group
  const int nblocks = (num_slots + 127) >> 7;          // 128-row blocks of the pool
  constexpr int kWinLog2 = K >= 16 ? 11 : 13;          // blocks per window: 2^18 or 2^20 rows
  const int wblocks = min(nblocks, 1 << kWinLog2);     // blocks of the largest window
  const int area = max(4 * wblocks, n);
  uint4* const bm = (uint4*)lds;                       // the window's bit map (a block per uint4), then its union rows
  uint32_t* const ubits = lds + area;                  // byte r: member bits of union entry r
  uint16_t* const pre = (uint16_t*)(ubits + ((n + 3) >> 2));   // the window's union rows before each block
  // entry e = i * P + tid of the members' lists laid end to end: member m = e / W and position
  // j = e - m W, the same for every group (as m << 16 | j, or -1 past the lists)
  const float rw = 1.0f / (float)W;
  auto entry = [&](int i) -> int32_t {
    const int e = i * P + tid;
    const int m = div_w(e, W, rw);
    return e < n ? (m << 16) | (e - m * W) : -1;
  };
  // the row loads' addresses are in range whatever the data (entries past the lists read the
  // last member's row and are masked), so all of them are in flight at once; the members'
  // counts are the same for every thread (scalar loads)
  int32_t raw[K], cnt_lane;                            // cnt_lane: member `lane`'s count (lanes < 8)
  auto load = [&](int g) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int32_t mj = entry(i);
      const int m = mj >> 16, j = mj & 0xffff;
      // the group's member m, or its last query for a short last group. With 16 entries per
      // thread the offsets from the group's first list are 32-bit (they span G * slots_stride
      // < 2^31 entries): the 64-bit addresses of all 16 loads in flight spilled registers (97
      // against 61 us for 8-query groups of 2,048 entries); with fewer entries the 64-bit form
      // is faster
      if constexpr (K >= 16) {
        const int mq = min(min(max(m, 0), G - 1), Q - 1 - g * G);
        raw[i] = mj >= 0 ? (slots + (int64_t)g * G * slots_stride)[(uint32_t)(mq * (int)slots_stride + j)] : -1;
      } else {
        const int q = min(g * G + min(max(m, 0), G - 1), Q - 1);
        raw[i] = mj >= 0 ? slots[(int64_t)q * slots_stride + j] : -1;
      }
    }
    // a vector load (a scalar one would be waited for at the next LDS barrier)
    const bool member = lane < G && g * G + lane < Q;
    cnt_lane = member ? (valid ? valid[g * G + lane] : W) : 0;
  };
  // with 16 entries per thread the next group's rows are not loaded ahead (registers)
  constexpr bool kAhead = K <= 8;
  int g = blockIdx.x;
  if (kAhead && g < groups) load(g);
  for (; g < groups; g += gridDim.x) {
    if (!kAhead) load(g);
    int32_t key[K];                                    // listed row | member << 24, or -1
    const int cnt_c = min(max(cnt_lane, 0), W);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int32_t mj = entry(i);
      const int m = mj >> 16, j = mj & 0xffff;
      const int lim = __shfl(cnt_c, m & 7, 64);
      key[i] = mj >= 0 && j < lim && raw[i] >= 0 && raw[i] < num_slots ? raw[i] | (m << 24) : -1;
    }
    if (kAhead && g + (int)gridDim.x < groups) load(g + gridDim.x);   // lands while this group is built
    for (int w = tid; w < ((n + 3) >> 2); w += P) ubits[w] = 0u;
    int base = 0;                                      // union rows of the windows before
    // (one window, known at compile time, for lists of up to 8,192 entries)
    const int nwin = K >= 16 ? (nblocks + (1 << kWinLog2) - 1) >> kWinLog2 : 1;
    for (int wi = 0; wi < nwin; ++wi) {
      // window wi: pool rows 128 b0 .., its keys' rows relative to it
      const int b0 = wi << kWinLog2;
      const int nbw = min(nblocks - b0, 1 << kWinLog2);
      const int per_wave = (nbw + kWaves - 1) / kWaves;  // blocks counted by each wave
      for (int b = tid; b < nbw; b += P) bm[b] = make_uint4(0u, 0u, 0u, 0u);
      lds_barrier();
      // a key of this window (every valid key with a single window)
      auto in_win = [&](int32_t k) { return K >= 16 ? k >= 0 && ((k & 0xffffff) >> (kWinLog2 + 7)) == wi : k >= 0; };
#pragma unroll
      for (int i = 0; i < K; ++i)
        if (in_win(key[i])) atomicOr(&lds[((key[i] & 0xffffff) - 128 * b0) >> 5], 1u << (key[i] & 31));
      lds_barrier();
      // set bits per block, and their prefix inside the wave's range: round k covers blocks
      // b_lo + 64k + lane (at most 8 rounds: a window of 2^20 rows is 8,192 blocks over 16 waves;
      // 2 for 2^18); the rounds' reads all go out first and their scans are independent
      constexpr int kRounds = 1 << (kWinLog2 - 10);
      const int b_lo = wv * per_wave, b_hi = min(b_lo + per_wave, nbw);
      int c[kRounds], incl[kRounds];
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int b = b_lo + 64 * k + lane;
        c[k] = 0;
        if (b < b_hi) {
          const uint4 x = bm[b];
          c[k] = __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
        }
      }
      int run = 0;
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        incl[k] = wave_inclusive_sum(c[k]) + run;
        run = __builtin_amdgcn_readlane(incl[k], 63);
      }
      if (lane == 0) wave_tot[wv] = run;
      lds_barrier();
      int off = 0, total = 0;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        off += k < wv ? wave_tot[k] : 0;
        total += wave_tot[k];
      }
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int b = b_lo + 64 * k + lane;
        if (b < b_hi) pre[b] = (uint16_t)(off + incl[k] - c[k]);
      }
      lds_barrier();
      // each listed entry's place in the union (the windows before, its block's count, plus the
      // set bits before it in the block), and its member's bit there
      // (with 16 entries per thread the place replaces the member in the key, window row | place
      // << 18, which holds in windows of 2^18 rows: the row's 18 bits are never all ones, so a
      // packed key is never -1; fewer entries keep the places apart)
      constexpr bool kPack = K >= 16;
      int place[kPack ? 1 : K];
      bool mine[kPack ? K : 1];                          // packed keys: this window's
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if constexpr (!kPack) place[i] = -1;
        if constexpr (kPack) mine[i] = in_win(key[i]);
        if (kPack ? mine[i] : in_win(key[i])) {
          const int r = (key[i] & 0xffffff) - 128 * b0, b = r >> 7, wq = (r >> 5) & 3;
          const uint4 x = bm[b];
          const uint32_t below = (1u << (r & 31)) - 1u;
          int pl = base + pre[b];
          pl += wq > 0 ? __popc(x.x) : __popc(x.x & below);
          pl += wq > 1 ? __popc(x.y) : (wq == 1 ? __popc(x.y & below) : 0);
          pl += wq > 2 ? __popc(x.z) : (wq == 2 ? __popc(x.z & below) : 0);
          pl += wq == 3 ? __popc(x.w & below) : 0;
          atomicOr(&ubits[pl >> 2], (1u << (key[i] >> 24)) << (8 * (pl & 3)));
          if constexpr (kPack) key[i] = r | (pl << 18);
          else place[i] = pl;
        }
      }
      lds_barrier();                                   // the bit map is read: it takes the window's rows
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if constexpr (kPack) {
          if (mine[i]) {
            lds[((uint32_t)key[i] >> 18) - base] = (uint32_t)key[i] & 0x3ffffu;
            key[i] = -1;                               // placed: no later window takes it
          }
        } else {
          if (place[i] >= 0) lds[place[i] - base] = (uint32_t)((key[i] & 0xffffff) - 128 * b0);
        }
      }
      lds_barrier();
      uint32_t* out = enc + (int64_t)g * enc_stride + base;
      for (int r = tid; r < total; r += P)
        out[r] = (lds[r] + 128 * b0) |
                 (((ubits[(base + r) >> 2] >> (8 * ((base + r) & 3))) & 0xffu) << SMLA_UNION_ROW_BITS);
      base += total;
      lds_barrier();                                   // before the next window or group clears the map
    }
    if (tid == 0) lens[g] = base;
  }
}

// Pools too large for the bit map: the group's keys (row << 3 | member, empty = 0xffffffff)
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
  const int t = threadIdx.x;
  uint32_t v[K];
  // the thread's keys before the sort: entries t, t + P, t + 2P, ... of the members' lists laid
  // end to end (any assignment sorts the same; this one makes each load instruction contiguous).
  // Entry e is position j = e - m W of member m = e / W. Every load address is in range
  // whatever the data (entries past the group's lists read the last member's row and are
  // masked afterwards), so all the loads are in flight at once.
  const float rw = 1.0f / (float)W;
  int32_t raw[K], lim[K], mj[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int e = i * P + t;
    const int m = div_w(e, W, rw), j = e - m * W;
    const int q = min(g * G + min(m, G - 1), Q - 1);
    raw[i] = slots[(int64_t)q * slots_stride + j];
    lim[i] = valid ? valid[q] : W;
    mj[i] = m < G && g * G + m < Q ? (m << 16) | j : -1;    // member and position, or not listed
  }
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int m = mj[i] >> 16, j = mj[i] & 0xffff;
    const int32_t r = raw[i];
    v[i] = mj[i] >= 0 && j < min(max(lim[i], 0), W) && r >= 0 && r < num_slots ? ((uint32_t)r << 3) | (uint32_t)m
                                                                                 : kEmpty;
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
  int total;
  int pos = block_exclusive_sum<P>(heads, wave_tot, total);
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

// A kernel's dynamic LDS limit, raised to `bytes` when a launch needs more than the limit set
// so far on the current device (each device keeps its own function attributes). Racing first
// calls may both set it; the larger value stays.
std::atomic<int32_t> lds_limit[5][64];

hipError_t allow_dynamic_lds(const void* kernel, int k, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int32_t>* lim = dev >= 0 && dev < 64 ? &lds_limit[k][dev] : nullptr;
  if (lim && lim->load(std::memory_order_relaxed) >= (int32_t)bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && lim) {
    int32_t cur = lim->load(std::memory_order_relaxed);
    while (cur < (int32_t)bytes && !lim->compare_exchange_weak(cur, (int32_t)bytes, std::memory_order_relaxed)) {
    }
  }
  return e;
}

}  // namespace

hipError_t launch_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                        int32_t Q, int32_t W, int32_t G, int64_t num_slots, uint32_t* enc,
                        int64_t enc_stride, int32_t* lens, int32_t cus, hipStream_t stream) {
  if (Q == 0) return hipSuccess;
  const int groups = (Q + G - 1) / G;
  const int n = G * W, nblocks = (int)((std::min<int64_t>(num_slots, kBitmapSlots) + 127) >> 7);
  // lists of more than 8,192 entries (16 per thread) map windows of 2^18 rows, which their
  // packed keys and two counting rounds assume; the others the whole pool
  const int wblocks = std::min(nblocks, n > 8192 ? 1 << 11 : 1 << 13);
  const size_t lds = (size_t)(std::max(4 * wblocks, n) + ((n + 3) >> 2)) * 4 + (size_t)wblocks * 2;
  // the window's bit map, the member bytes and the block counts must fit one compute unit's
  // LDS beside the kernel's own; a group's list entries must sit within 2^31 entries of its
  // first (32-bit offsets)
  if (num_slots <= kBitmapSlots && lds + 1024 <= 160u * 1024u && (int64_t)G * slots_stride < ((int64_t)1 << 31)) {
    // as many workgroups as fit the compute units at once (registers and LDS decide)
#define SMLA_UNION_BITMAP(K)                                                                                        \
  do {                                                                                                              \
    hipError_t e = allow_dynamic_lds((const void*)union_bitmap_kernel<K>, __builtin_ctz(K), lds);                  \
    if (e != hipSuccess) return e;                                                                                  \
    int per_cu = 0;                                                                                                 \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)union_bitmap_kernel<K>, kBitmapThreads, \
                                                     lds);                                                          \
    if (e != hipSuccess) return e;                                                                                  \
    const int grid = (int)std::min<int64_t>(groups, (int64_t)std::max(1, cus) * std::max(1, per_cu));               \
    hipLaunchKernelGGL((union_bitmap_kernel<K>), dim3(grid), dim3(kBitmapThreads), lds, stream, slots, slots_stride, \
                       valid, Q, W, G, (int32_t)num_slots, groups, enc, enc_stride, lens);                          \
  } while (0)
    if (n <= 1024) SMLA_UNION_BITMAP(1);
    else if (n <= 2048) SMLA_UNION_BITMAP(2);
    else if (n <= 4096) SMLA_UNION_BITMAP(4);
    else if (n <= 8192) SMLA_UNION_BITMAP(8);
    else SMLA_UNION_BITMAP(16);                  // 16384, the largest G * W the ABI accepts
#undef SMLA_UNION_BITMAP
    return hipGetLastError();
  }
  int keys = 256;                                  // the sort's key count: G * W rounded up to a power of two
  while (keys < G * W) keys <<= 1;
#define SMLA_UNION_SORT(P, K)                                                                                        \
  hipLaunchKernelGGL((union_sort_kernel<P, K>), dim3(groups), dim3(P), 0, stream, slots, slots_stride, valid, Q, W, G, \
                     num_slots, enc, enc_stride, lens)
  switch (keys) {
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
