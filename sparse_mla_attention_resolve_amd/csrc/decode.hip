// Split decode attention over a block table.
//
// Stage 1 (one workgroup per token, block of 64 heads and split) walks the split's rows in
// chunks of 32: it gathers the chunk's 576-wide rows from the pool into LDS, computes the
// scores of the block's 64 heads against them with bf16 MFMA (every head of the token meets
// each gathered row; the scores are computed transposed, rows on the M dimension and heads
// on N), keeps a running max and sum per head (online softmax), and accumulates P * V with
// MFMA, V being the first 512 columns of the same rows. The splits of a token are merged by
// LSE at the end of stage 1 (bf16 q), or by stage 2 (IBM Triton paged-attention explainer,
// section 4 table: "Q-Block" for stacking the heads that share a KV row, "Parallel Tiled
// Softmax" for the split and merge).
//
// The block table is either resolved slots (page size 1, the virtual block table of
// The Virtual Block Table: Reusing Triton MLA for Sparse Attention on Blackwell GPUs,
// "The Breakthrough") or page ids (page size P > 1, the dense paged walk of "The
// Investigation"). fp8 caches are dequantised in the kernel: each gathered chunk's e4m3
// codes convert to bf16 exactly, once per workgroup, into a staging tile that the bf16 MFMA
// loop reads; the per-row scale multiplies the latent part of the score and the softmax
// weight that meets the row's values.
#include "stage1_common.h"

namespace smla {

namespace {

constexpr int kThreads = 256;

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

// Stage 1 workgroup: 8 waves, two per SIMD. Wave w = (hq, x) with hq = w & 3, x = w >> 2
// owns heads 16hq .. 16hq+15; for the scores it takes rows 16x .. 16x+15 of each chunk, for
// the output it takes latent columns 256x .. 256x+255. Its partner w ^ 4 holds the other half.
constexpr int kS1Waves = 8;
constexpr int kS1Threads = 64 * kS1Waves;
#ifndef SMLA_PV_IN_A
#define SMLA_PV_IN_A 2
#endif
constexpr int kPvA = SMLA_PV_IN_A;          // P V tiles of chunk ci computed with the scores of chunk ci + 1
#ifndef SMLA_PV_PUB
#define SMLA_PV_PUB 6
#endif
constexpr int kPvPub = SMLA_PV_PUB;         // P V tiles of chunk ci computed while chunk ci + 1's weights are formed
#ifndef SMLA_PV_FP8
#define SMLA_PV_FP8 4
#endif
constexpr int kPvF = SMLA_PV_FP8;           // fp8: P V tiles of chunk ci computed while chunk ci + 1 is converted

// Two floats as nearest bf16 (ties to even), lo in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The balanced plan of a dense paged decode of tv <= 64 virtual tokens (64-head blocks; virtual
// token v is block v / T of token v % T), computed by one wave from the lengths alone, lane v for
// token v: token v gets n_v = max(1, ceil(len_v / r)) splits of at most r rows, numbered
// consecutively in token order from base. r (whole chunks, at least min_rows) is
// ceil(total / (cus - tv)), at which the splits always fit the compute units (sum n_v <=
// total / r + tv); when that is more than one segment of kMaxSplitRows rows, r is instead the
// fewest rows whose splits fit: a binary search down to ceil(total / cus), since the count only
// falls as r grows. (Below a segment, more splits than that would add more merge work than
// balance; above it, the rounding of ceil(len_v / r) can leave a quarter of the units idle.)
// A split longer than kMaxSplitRows rows builds its slots a block of that many at a time
// (SEGS). Stage 1 and stage 2 compute the same plan. Returns the total number of splits
// (wave-uniform).
struct BalancedPlan {
  int r, base, n, total;
};
// the sum over the wave's 64 lanes (all active), in every lane: DPP moves, no LDS
__device__ __forceinline__ int wave_sum_i(int x) { return __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63); }
// ceil(a / b) for a >= 0, b >= 8 and a + b <= 2^25: the fp32 reciprocal estimate (relative
// error ~2^-22) puts the truncated quotient within one of the true one, which one step each way
// corrects
__device__ __forceinline__ int ceil_div_small(int a, int b) {
  const int num = a + b - 1;
  int q = (int)((float)num * __builtin_amdgcn_rcpf((float)b));
  q -= q * b > num ? 1 : 0;
  q += (q + 1) * b <= num ? 1 : 0;
  return q;
}
__device__ __forceinline__ BalancedPlan balanced_plan(const int32_t* lens, int T, int hblocks, int max_len, int cus,
                                                      int min_rows, int v) {
  const int tv = T * hblocks;
  int ln = 0;
  if (v < tv) {
    const int l = lens[v % T];
    ln = l < 0 ? 0 : (l > max_len ? max_len : l);
  }
  const int tot = wave_sum_i(ln);
  auto splits_of = [&](int r) { return v < tv ? max(1, ceil_div_small(ln, r)) : 0; };
  const int cmin = (min_rows + kChunk - 1) / kChunk;       // in chunks
  int hi = max(cmin, ceil_div_small(tot, (cus - tv) * kChunk));
  int lo = hi * kChunk <= kMaxSplitRows ? hi : max(cmin, ceil_div_small(tot, cus * kChunk));
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (wave_sum_i(splits_of(mid * kChunk)) <= cus) hi = mid;
    else lo = mid + 1;
  }
  const int r = hi * kChunk;
  const int n = splits_of(r);
  const int incl = wave_inclusive_sum(n);
  return BalancedPlan{r, incl - n, n, __builtin_amdgcn_readlane(incl, 63)};
}

// Workgroup id -> (token, split). Workgroups are dispatched to the 8 XCDs round robin;
// when T is a multiple of 8 every split of a token runs on one XCD, so the token's partial
// results stay in that XCD's L2 for stage 2, which uses the same token -> XCD rule.
__device__ __forceinline__ void stage1_coords(int b, int T, int S, int& t, int& s) {
  if ((T & 7) == 0) {
    const int i = b >> 3;
    t = (b & 7) + 8 * (i / S);
    s = i % S;
  } else {
    t = b / S;
    s = b % S;
  }
}

// One step of wave (hq, x) over chunks of bf16 rows: the scores of one chunk's rows
// 16x .. 16x+15 (S^T tile: lane (g, c) gets rows 16x + 4g + v of head 16hq + c; 18 MFMAs on two
// accumulator chains) and / or O += P V over another chunk's columns 256x .. 256x+255 (16 MFMAs,
// one per 16-column tile), interleaved so that the matrix unit always has independent work
// while the operand reads run kAhead steps ahead. With ROPE_APART the scores' latent part
// (dims 0 .. 511) goes to sl and the rotary part to sr (an fp8 cache scales the latent part
// alone); otherwise sl holds both. after_step(k) runs after step k's MFMAs are issued (the
// caller spreads its gathers of a later chunk over the steps).
template <bool DO_S, bool DO_PV, bool ROPE_APART, typename Hook, int PV0 = 0, int PV1 = 16>
__device__ __forceinline__ void chunk_step(const char* kbS, const char* kbV, const Offsets& off,
                                           const bf16x8 (&qf)[kQLoads], f32x4& sl, f32x4& sr, const bf16x8& pa,
                                           f32x4 (&oacc)[16], Hook&& after_step) {
  // P V tiles PV0 .. PV1 - 1 (at steps 0 .. PV1 - PV0 - 1)
  constexpr int kNPV = DO_PV ? PV1 - PV0 : 0;
  constexpr int kSteps = DO_S ? 18 : kNPV;
  f32x4 acc[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                  f32x4{0.f, 0.f, 0.f, 0.f}};
  auto kread = [&](int ks) -> uint4 { return *(const uint4*)(kbS + off.ka[ks & 1] + 64 * ks); };
  auto vread = [&](int nt) -> uint4 {
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(kbV + off.vo[nt & 3] + 128 * (nt >> 2)));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(kbV + off.vo[4 + (nt & 3)] + 128 * (nt >> 2)));
    return __builtin_bit_cast(uint4, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  uint4 kq[kAhead + 1], vq[kAhead + 1];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    if constexpr (DO_S) kq[i] = kread(i);
    if constexpr (DO_PV) { if (i < kNPV) vq[i] = vread(PV0 + i); }
  }
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    if constexpr (DO_S) {
      if (k + kAhead < 18) kq[(k + kAhead) % (kAhead + 1)] = kread(k + kAhead);
      const int ai = (ROPE_APART && k >= 16 ? 2 : 0) + (k & 1);
      acc[ai] = mfma16x16x32(as_bf16x8(kq[k % (kAhead + 1)]), qf[k], acc[ai]);
    }
    if constexpr (DO_PV) {
      if (k < kNPV) {
        if (k + kAhead < kNPV) vq[(k + kAhead) % (kAhead + 1)] = vread(PV0 + k + kAhead);
        oacc[PV0 + k] = mfma16x16x32(pa, as_bf16x8(vq[k % (kAhead + 1)]), oacc[PV0 + k]);
      }
    }
    after_step(k);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (DO_S) {
    sl = acc[0] + acc[1];
    if constexpr (ROPE_APART) sr = acc[2] + acc[3];
  }
}

// ---- merge of a token's splits inside stage 1
//
// The split workgroups of a token write their partials with agent-scope atomic stores (sc1:
// written through to the device-wide coherence point) and read the other workgroups'
// partials with agent-coherent loads (sc1: served from that point, never from a stale L1 or
// L2 line). The order between a writer's stores and a reader's loads is kept by the
// instructions themselves rather than by cache maintenance:
//   - every thread waits for its own stores to complete (s_waitcnt vmcnt(0), an asm statement
//     the compiler cannot move memory operations across) before the workgroup barrier that
//     precedes the workgroup's ticket, so a ticket is only ever counted after its partials
//     sit at the coherence point;
//   - a reader issues its loads only after it has read every ticket, behind a workgroup
//     barrier (the compiler hoists no load above it; the hardware does not issue loads ahead
//     of the instructions before them).
// The memory model's own form of this, an agent-scope release on the ticket and an acquire
// before the loads, compiles on gfx950 to a write-back of the whole L2 (buffer_wbl2) and an
// invalidate of it (buffer_inv); measured on the batch-32 bf16 decode step, the release adds
// 1.8 us, the acquire 2.8 us, both 4.3 us (15% of the step), for no data that is not already
// written through and read from the coherence point.
//
// Word of token t (zero on entry, zero again when its last workgroup leaves):
//   bits 0 .. 8    tickets taken (arrivals), bits 9 .. 17 departures,
//   bits 18 .. 25  parts given up by tickets 0 .. 7.
// The merge has 8 parts (head quarter x column half), owned by tickets 0 .. 7 (parts_of).
// A ticket holder waits a bounded time for the remaining arrivals and then merges its parts;
// when the time runs out it gives them up with one atomic add, which also tells it whether
// the last arrival has already come (then it merges them after all). The last arrival never
// waits: it merges its own parts and every part given up before it came.
constexpr uint32_t kArrMask = 0x1ff;
constexpr int kExitShift = 9, kGiveUpShift = 18;
constexpr int kBufFlags = 0x00020000;       // buffer descriptor word 3: 32-bit data format
constexpr int kSc1 = 16;                    // cache-policy operand of buffer loads: sc1

// The merge parts of the workgroup that arrived q-th among nact: a contiguous range of the
// eight (one part each from 8 splits on, none for q >= 8), so that the two column halves of a
// head quarter usually fall to one workgroup, which merges them in one pass.
__device__ __forceinline__ uint32_t parts_of(int q, int nact) {
  if (nact >= 8) return q < 8 ? 1u << q : 0u;
  const int p0 = (8 * q + nact - 1) / nact, p1 = (8 * (q + 1) + nact - 1) / nact;
  return ((1u << p1) - 1u) & ~((1u << p0) - 1u);
}

// Part p (0 .. 7) of token t's merge: heads 16(p >> 1) .. +15 x columns 256(p & 1) .. +255,
// which are packed entries 1024p .. 1024p + 1023 of every split's partial. Thread i merges
// entries 1024p + 2i and + 1: heads hb .. hb + 3 at columns col and col + 1 (the entries of
// lanes c and c + 1 of one group g). Per batch of eight splits, 128 threads fetch the
// part's 16 x 8 LSEs into LDS (`scratch`, 128 floats) while every thread has its eight
// 16-byte slices in flight; the weights keep a running maximum:
// O = sum_s exp(lse_s - lse) O_s with lse = log sum_s exp(lse_s).
// NP = 2 merges parts p and p + 1 (p even: the two column halves of one head quarter, entries
// 1024 further on, columns 256 further on) with the same LSEs and weights.
// pbase is the first of the token's partials (its splits' partials are consecutive), tr the
// token and hbase + hb its output heads, of which the first hv of the 64 exist.
template <int NP>
__device__ __forceinline__ void merge_part(const Stage1Args& a, int64_t pbase, int tr, int hbase, int hv, int nact,
                                           int p, int tid, float* scratch) {
  static_assert(NP == 1 || NP == 2, "one part or a head quarter's two");
  constexpr int kBatch = 8;
  const int j = 1024 * p + 2 * tid;
  const int lanep = j & 63, ntp = (j >> 6) & 15;
  const int hp = 4 * (lanep >> 4);                       // head offset inside the part's 16
  const int hb = 16 * (p >> 1) + hp;
  const int col = 256 * (p & 1) + 16 * ntp + (lanep & 15);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.part_o + pbase * (kHeads * kLatent)), (short)0, 0x7fffffff, kBufFlags);
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.part_lse + pbase * kHeads), (short)0, 0x7fffffff, kBufFlags);
  float mx[4], ws[4], acc[NP][4][2];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    mx[v] = -INFINITY;
    ws[v] = 0.f;
#pragma unroll
    for (int n = 0; n < NP; ++n) acc[n][v][0] = acc[n][v][1] = 0.f;
  }
  for (int s0 = 0; s0 < nact; s0 += kBatch) {
    // (every thread loads an in-range LSE, unconditionally, so that no wait for it comes
    // before the slices go out; only threads < 128 keep theirs)
    const int ls = s0 + ((tid >> 4) & (kBatch - 1));
    const float lv = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rl, ((ls < nact ? ls : s0) * kHeads + 16 * (p >> 1) + (tid & 15)) * 4, 0, kSc1));
    uint4 o[NP][kBatch];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const int sp = s0 + jj < nact ? s0 + jj : s0;
        o[n][jj] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(ro, sp * (kHeads * kLatent * 2) + 8 * (j + 1024 * n), 0, kSc1));
      }
    __syncthreads();                                     // the previous batch's LSEs are read
    if (tid < 16 * kBatch) scratch[tid] = ls < nact ? lv * kLog2e : -INFINITY;   // base 2 from here on
    __syncthreads();
    float4 l[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) l[jj] = *(const float4*)(scratch + 16 * jj + hp);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float bm = mx[v];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) bm = fmaxf(bm, ((const float*)&l[jj])[v]);
      if (bm == -INFINITY) continue;                     // nothing but empty splits so far
      const float r = __builtin_amdgcn_exp2f(mx[v] - bm);   // 0 on the first non-empty pass
      ws[v] *= r;
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        acc[n][v][0] *= r;
        acc[n][v][1] *= r;
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const float lw = ((const float*)&l[jj])[v];
        const float wgt = lw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lw - bm);
        ws[v] += wgt;
        // entry 2i: words x, y = heads (0, 1), (2, 3) at col; entry 2i + 1: z, w at col + 1.
        // Explicit fused multiply-adds: a part merged alone (NP = 1) or with its neighbour
        // (NP = 2) must round the same, since which of the two runs depends on arrival order
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          const uint32_t w0 = v < 2 ? o[n][jj].x : o[n][jj].y, w1 = v < 2 ? o[n][jj].z : o[n][jj].w;
          acc[n][v][0] = __builtin_fmaf(wgt, bf16_to_f32((v & 1) ? (w0 >> 16) : (w0 & 0xffffu)), acc[n][v][0]);
          acc[n][v][1] = __builtin_fmaf(wgt, bf16_to_f32((v & 1) ? (w1 >> 16) : (w1 & 0xffffu)), acc[n][v][1]);
        }
      }
      mx[v] = bm;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (hb + v >= hv) continue;                         // a head slot past the block's heads
    const float inv = ws[v] > 0.f ? 1.0f / ws[v] : 0.f;
    uint32_t* o =
        (uint32_t*)((uint16_t*)a.out + (int64_t)tr * a.out_tok_stride + (int64_t)(hbase + hb + v) * a.out_head_stride + col);
#pragma unroll
    for (int n = 0; n < NP; ++n) o[128 * n] = cvt_bf16x2(acc[n][v][0] * inv, acc[n][v][1] * inv);
    if (a.lse && (p & 1) == 0 && ntp == 0 && (lanep & 15) == 0)
      a.lse[(int64_t)tr * a.lse_tok_stride + hbase + hb + v] = ws[v] > 0.f ? (mx[v] + log2f(ws[v])) * kLn2 : -INFINITY;
  }
}

// Called by every active split workgroup of virtual token t (token tr, heads hbase .. hbase + hv
// - 1) once its partial is stored, with nact >= 2 the token's active splits.
__device__ __forceinline__ void merge_splits(const Stage1Args& a, int t, int64_t pbase, int tr, int hbase, int hv,
                                             int nact, int wait_ticks, int tid, float* scratch) {
  __shared__ uint32_t bcast;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");       // this thread's partial stores are complete
  __syncthreads();
  uint32_t* const word = a.sync + (int64_t)t * kSyncStride;
  if (tid == 0) bcast = __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t old = bcast;
  const int q = (int)(old & kArrMask);
  uint32_t todo = 0;
  if (q == nact - 1) {
    todo = parts_of(q, nact);
    const uint32_t gave_up = (old >> kGiveUpShift) & 0xffu;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((gave_up >> k) & 1u) todo |= parts_of(k, nact);
  } else if (q < 8) {
    __syncthreads();                                           // every thread has read bcast
    if (tid == 0) {
      uint32_t seen = 0;
      if (wait_ticks > 0) {
        const uint64_t t0 = wall_clock64();
        do {
          if ((__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kArrMask) >= (uint32_t)nact) {
            seen = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        } while (wall_clock64() - t0 < (uint64_t)wait_ticks);
      }
      if (!seen) {
        const uint32_t o2 = __hip_atomic_fetch_add(word, 1u << (kGiveUpShift + q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        seen = (o2 & kArrMask) >= (uint32_t)nact;             // the last arrival came first: keep the parts
      }
      bcast = seen;
    }
    __syncthreads();
    if (bcast) todo = parts_of(q, nact);
  }
#pragma unroll 1
  for (int k = 0; k < 8; ++k) {
    if (!((todo >> k) & 1u)) continue;
    if ((k & 1) == 0 && ((todo >> (k + 1)) & 1u)) {
      merge_part<2>(a, pbase, tr, hbase, hv, nact, k, tid, scratch);   // both column halves of a head quarter
      ++k;
    } else {
      merge_part<1>(a, pbase, tr, hbase, hv, nact, k, tid, scratch);
    }
  }
  if (tid == 0) {
    const uint32_t o3 = __hip_atomic_fetch_add(word, 1u << kExitShift, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (((o3 >> kExitShift) & kArrMask) == (uint32_t)nact - 1)   // everyone else is done with the word
      __hip_atomic_store(word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Stage 1. The scores are computed transposed, S^T = K Q^T (chunk rows are the M dimension
// of a 16x16x32 MFMA tile, heads the N dimension, K = 576), so that lane (g, c) holds head
// c's scores for rows 4g .. 4g+3 of its half. Each wave turns them into weights and the two
// partners swap those through LDS, after which each lane holds head c's eight weights, for its
// own rows 16x + 4g + v and then its partner's: the softmax statistics need only cross-lane
// moves inside the wave, and the eight weights are the A operand of the P V product (16x16x32,
// K = the chunk's 32 rows taken in that order), whose B operand the transposing LDS reads
// fetch in the same row order. The loop is software pipelined: while it accumulates P V for
// chunk ci it computes the scores and weights of chunk ci + 1.

// SEGS (decode): a split may be longer than one block of kMaxSplitRows rows, which only the
// balanced plan makes; the other decode launches keep the plan and the block pipeline out of
// their code.
template <int KV, bool UNION, bool BYIDX, bool SEGS>
__global__ void __launch_bounds__(kS1Threads, 1) decode_stage1_mfma(Stage1Args a) {
  using L = Lay<KV>;
  constexpr int kRowBytes = L::kUnits * 16;
  constexpr int kChunkBytes = kChunk * kRowBytes;
  constexpr int kInstr = kChunk * L::kUnits / 64;           // 16-byte x 64-lane copies per chunk: 36 / 20
  static_assert(kChunk * L::kUnits % 64 == 0, "a chunk must be whole copy instructions");
  constexpr int kLoadsHi = kInstr / kS1Waves + 1, kLoadsLo = kInstr / kS1Waves;
  constexpr int kHiWaves = kInstr % kS1Waves;               // waves 0 .. kHiWaves-1 issue one more copy
  constexpr int kNBuf = L::kNBuf;
  constexpr bool kFp8 = KV == SMLA_FP8_E4M3;
  __shared__ __attribute__((aligned(16))) char kvbuf[kNBuf][kChunkBytes];
  // fp8: each chunk's rows converted to bf16 rows (the layout of a bf16 chunk), two chunks
  constexpr int kStgBytes = kChunk * Lay<SMLA_BF16>::kUnits * 16;
  __shared__ __attribute__((aligned(16))) char stg[kFp8 ? 2 : 1][kFp8 ? kStgBytes : 16];
  // SEGS: two blocks of kMaxSplitRows slots, the next block built while the current one runs
  constexpr int kSlotRows = SEGS ? 2 * kMaxSplitRows : kMaxSplitRows;
  __shared__ __attribute__((aligned(16))) int32_t slot_s[kSlotRows];
  __shared__ int32_t page_s[kMaxSplitRows / 2 + 64];     // page ids of a split (page size >= 2)
  __shared__ __attribute__((aligned(16))) float scale_s[kFp8 ? kSlotRows : 4];
  __shared__ uint2 px[kS1Waves][64];                       // weights (bf16) swapped between partners
  __shared__ float mx[kS1Waves][16];                       // the reference each wave's weights are relative to
  __shared__ int fx[kS1Waves];                             // 1: that reference is the running max
  __shared__ float lx[kS1Waves][16];                       // the partners' sums, at the end
  __shared__ int wcnt[kMaxSplitRows / kS1Threads][kS1Waves];   // union mode: kept entries per wave

  // t, s: the (virtual) token and split; rps rows per split, pbase the token's first partial,
  // smax the cap on a token's splits
  int t, s, rps = a.rows_per_split, smax = a.S, wait_ticks = a.wait_ticks;
  int64_t pbase;
  if constexpr (!UNION && SEGS) {                         // launched for a balanced plan (a.balanced)
    // Splits planned from the lengths (a dense paged decode of at most 64 tokens, whose
    // contexts may differ widely): rows per split from the launch's total rows, so that every
    // token's splits fit the compute units at once (at least min_rows, whole chunks, in
    // blocks of kMaxSplitRows rows); token v gets ceil(len_v / rows) splits, at least one
    // (which writes an empty token's output); workgroup b takes the b-th split in token order,
    // or leaves past the last. Wave 0 plans, lane v for token v.
    __shared__ int bplan[5];
    if (threadIdx.x < 64) {
      const int v = threadIdx.x, b = blockIdx.x;
      const BalancedPlan bp = balanced_plan(a.lens, a.T, a.hblocks, a.max_len, a.cus, a.min_rows, v);
      const bool mine = bp.n > 0 && b >= bp.base && b < bp.base + bp.n;
      const uint64_t m = __ballot(mine);
      if (v == 0) {
        bplan[0] = m ? __builtin_ffsll((long long)m) - 1 : -1;
        bplan[2] = bp.r;
        // the splits are the launch's first `total` workgroups, dispatched before the ones that
        // leave at once: only when they fit the compute units together may one wait for another
        bplan[4] = bp.total <= a.cus ? a.wait_ticks : 0;
      }
      if (mine) {
        bplan[1] = b - bp.base;
        bplan[3] = bp.base;
      }
    }
    __syncthreads();
    t = bplan[0];
    if (t < 0) return;                                     // past the last split
    s = bplan[1];
    rps = bplan[2];
    pbase = bplan[3];
    smax = kMaxSplitRows;                                  // no cap: ceil(len / rps) splits
    wait_ticks = bplan[4];
  } else {
    stage1_coords(blockIdx.x, UNION ? a.T : a.T * a.hblocks, a.S, t, s);
    pbase = (int64_t)t * a.S;
  }
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform, kept in an SGPR
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int hq = w & 3, x = w >> 2;
  const int h0 = 16 * hq;
  // waves issuing kLoadsHi copies per chunk (the others kLoadsLo): the first kHiWaves
  const bool hi = w < kHiWaves;

  // ---- prologue. What the first gathers need goes out as early as it can:
  //   - at once (it needs only the kernel's arguments): the split's table entries
  //     table[t][e0 .. e0 + n_ent) (slots when the page size is 1, page ids otherwise) into
  //     slot_s / page_s; for a page-mapped table, the guessed request's page-table row into
  //     ring slot 1 when the row fits there; then the scalar loads of the token's length and
  //     request and the guessed request's context length;
  //   - once the request is known, if the guess was wrong: its context length and row.
  // All of it lands before the slots are built, so that building them touches LDS only (a
  // register that a global load may still be writing would make the compiler wait for
  // every copy in flight, since it does not see them). Decode issues q right behind it and
  // leaves q in flight meanwhile; union mode issues q first.
  const int lp = a.log2_page;
  const int r0 = s * rps;
  const bool mapped = !UNION && a.mapped != 0;          // union mode never maps
  constexpr bool umode = UNION;                         // a.union_G > 0
  // union mode: heads per query, queries per workgroup, workgroups per group, this
  // workgroup's group and first member; head hh of the workgroup is head hh % uH of query
  // grp * G + m0 + hh / uH
  const int uH = umode ? a.H : kHeads;
  const int mpw = kHeads / uH;
  const int wgpg = umode ? a.union_G / mpw : 1;
  const int grp = umode ? t / wgpg : t;
  const int m0 = umode ? (t % wgpg) * mpw : 0;
  // decode: t is a virtual token, tr its token, hbk its block of 64 heads, hv the block's
  // real heads
  const int tr = umode ? t : t % a.T;
  const int hbk = umode ? 0 : t / a.T;
  const int hv = umode ? kHeads : min(kHeads, a.H - kHeads * hbk);
  auto tok_of = [&](int hh) { return umode ? grp * a.union_G + m0 + hh / uH : tr; };
  auto head_of = [&](int hh) { return umode ? hh % uH : kHeads * hbk + min(hh, hv - 1); };
  auto writes = [&](int hh) { return umode ? tok_of(hh) < a.T : hh < hv; };   // head slot hh has an output
  if (umode && tok_of(0) >= a.T) return;               // a short last group's missing members
  const int trow_id = umode ? grp : tr;                // the table row (union mode: the group's)
  const int32_t* trow = a.table + (int64_t)trow_id * a.table_stride;
  const int e0 = r0 >> lp;
  // the first block's entries (only a balanced plan makes splits of more than one block of
  // kMaxSplitRows rows: their later page ids are copied block by block)
  const int rps1 = min(rps, kMaxSplitRows);
  const int n_ent = lp == 0 ? min(rps1, a.max_len - r0) : min((r0 + rps1 - 1) >> lp, a.table_width - 1) - e0 + 1;
  // q's staging: bf16, ring slots 2 ..; fp8, the two staging tiles
  static_assert(kFp8 ? 2 * kStgBytes >= 4 * kQLoads * 1024 : (kNBuf - 2) * kChunkBytes >= 4 * kQLoads * 1024,
                "q must fit its staging");
  char* const qlds = (kFp8 ? stg[0] : kvbuf[2]) + hq * (kQLoads * 1024);
  int32_t* const prow_lds = (int32_t*)kvbuf[1];
  const bool row_in_lds = a.map_pt_width <= kChunkBytes / 4;
  int32_t req = -1, seq = 0;
  int len;                                     // the token's length, clamped to max_len
  // q, in the order the lanes read it back (head quarter hq: piece ks of lane (g, c) = head
  // 16hq + c, dims 32ks + 8g .. +7) into its staging (wave (hq, x) copies pieces 9x .. 9x+8
  // of quarter hq)
  auto copy_q = [&]() {
    const int qt = min(tok_of(h0 + c), a.T - 1);       // a short group repeats its last query
    const uint16_t* qh = a.q + (int64_t)qt * a.q_tok_stride + (int64_t)head_of(h0 + c) * a.q_head_stride + 8 * g;
#pragma unroll
    for (int k = 0; k < kQLoads / 2; ++k) {
      const int ks = 9 * x + k;
      dma16(qh + 32 * ks, qlds + ks * 1024);
    }
  };
  {
    if constexpr (UNION) copy_q();              // union mode: q lands with the entries
    int32_t* ent = lp == 0 ? slot_s : page_s;
    for (int k = w; k * 64 < n_ent; k += kS1Waves) {
      const int e = k * 64 + lane;
      dma4(e < n_ent ? (const void*)(trow + e0 + e) : (const void*)kZeroRow, (char*)(ent + k * 64));
    }
    // the page-table row of request r into ring slot 1
    auto copy_ptrow = [&](int r) {
      const int32_t* ptrow = a.map_pt + (int64_t)r * a.map_pt_stride;
      for (int k = w; k * 64 < a.map_pt_width; k += kS1Waves) {
        const int e = k * 64 + lane;
        dma4(e < a.map_pt_width ? (const void*)(ptrow + e) : (const void*)kZeroRow, (char*)(prow_lds + k * 64));
      }
    };
    // In a decode batch every request has one token and token t usually belongs to request
    // t: that request's page-table row and context length go out at once, with the entries,
    // instead of one round trip later behind the token's request id. A token of another
    // request fetches its own once the guessed ones have landed.
    const bool guess = mapped && trow_id < a.map_R;
    if (guess && row_in_lds) copy_ptrow(trow_id);
    // decode: q goes out right behind the entries (it depends on the token alone) and stays
    // in flight while the slots are built: the waits below cover the copies issued before q
    if constexpr (!UNION) copy_q();
    // The token's length and request id are cold loads. They go out only now, behind the
    // copies (the empty asm keeps the compiler from hoisting them), since a copy whose
    // address needs a kernel argument would otherwise wait for them too: scalar loads
    // complete out of order, so any wait for one waits for all. They are scalar loads
    // through the constant address space (the arrays are read-only here): as vector loads
    // behind the copies their first use would wait for every copy in flight.
    using cint = const __attribute__((address_space(4))) int32_t;
    int row = trow_id;
    __asm__ volatile("" : "+s"(row));
    int len_raw = ((cint*)a.lens)[row];
    int req_raw = mapped ? ((cint*)a.map_req)[row] : -1;
    int32_t seq_guess = guess ? ((cint*)a.map_seq)[row] : 0;
    __asm__ volatile("" : "+s"(len_raw), "+s"(req_raw), "+s"(seq_guess));   // all three in flight together
    len = len_raw < 0 ? 0 : (len_raw > a.max_len ? a.max_len : len_raw);
    bool reissue = false;
    if (mapped) {
      if (req_raw >= 0 && req_raw < a.map_R) {
        req = req_raw;
        seq = req == trow_id ? seq_guess : ((cint*)a.map_seq)[req];
      }
      reissue = row_in_lds && !(guess && req == trow_id) && req >= 0;
    }
    if (reissue) {
      wait_vmcnt<0>();                          // the guessed row's copies land first: both write the same LDS
      copy_ptrow(req);
      wait_vmcnt<0>();
    } else if constexpr (!UNION) {
      wait_vmcnt<kQLoads / 2>();
    } else {
      wait_vmcnt<0>();
    }
  }
  if (r0 >= len) {                              // inactive split: no merge reads it
    wait_vmcnt<0>();                            // no copy may land after the workgroup is gone
    if ((a.sync != nullptr || umode) && len == 0 && s == 0) {
      // a token with no rows: zero output and lse -inf (stage 2 would write them otherwise)
      for (int i = tid; i < kHeads * kLatent; i += kS1Threads) {
        const int hh = i >> 9;
        if (writes(hh))
          ((uint16_t*)a.out)[(int64_t)tok_of(hh) * a.out_tok_stride + (int64_t)head_of(hh) * a.out_head_stride + (i & 511)] = 0;
      }
      if (a.lse && tid < kHeads && writes(tid))
        a.lse[(int64_t)tok_of(tid) * a.lse_tok_stride + head_of(tid)] = -INFINITY;
    }
    return;
  }
  const int r1 = min(r0 + rps, len);
  lds_barrier();

  bf16x8 qf[kQLoads];                           // decode: loaded with the first chunks
  if constexpr (UNION) {
#pragma unroll
    for (int ks = 0; ks < kQLoads; ++ks) qf[ks] = as_bf16x8(*(const uint4*)(qlds + ks * 1024 + lane * 16));
  }

  // plane bases and strides as scalars (a per-lane choice between two fields of the
  // argument struct would otherwise become a memory load)
  const char* const lat8 = (const char*)a.kv.lat8;
  const char* const rope16_m32 = (const char*)a.kv.rope16 - 32 * 16;
  // row strides fit 32 bits (a row is at most a few KB), so slot * stride is one 32x32->64 multiply
  const uint32_t lat8_stride32 = (uint32_t)a.kv.lat8_stride, rope16_stride32 = (uint32_t)a.kv.rope16_stride;
  const uint32_t row_stride32 = (uint32_t)a.kv.row_stride;
  // BYIDX (a pool of at most 2^32 bytes whose gathered units sit in one row: bf16, or fp8
  // with the rotary part right behind the codes in the same stride, as gathers_by_index
  // decides): the rows are read by index through a buffer resource, so that a copy takes the
  // slot as it is and a masked row (index -1) reads zeros. Otherwise each lane forms its
  // 64-bit address.
  const char* const rbase = kFp8 ? lat8 : (const char*)a.kv.rows;
  const uint32_t rstride = kFp8 ? lat8_stride32 : row_stride32;
  const u32x4 rrsrc = row_rsrc(rbase, rstride, (uint32_t)a.kv.num_slots);

  // gather chunk ci into ring slot ci % kNBuf: copy instruction i = 8k + w of a chunk puts
  // the chunk's 16-byte units 64i .. 64i+63 (row-major, unit positions swizzled) at bytes
  // 1024i of the slot. Each lane's (row, stored unit) pairs are the same for every chunk;
  // masked rows gather from the zero row.
  int32_t lpos[kLoadsHi];
#pragma unroll
  for (int k = 0; k < kLoadsHi; ++k) {
    const int pos = (k * kS1Waves + w) * 64 + lane;
    const int row = pos / L::kUnits, unit = swz<KV>(row, pos % L::kUnits);   // the swizzle is an involution
    lpos[k] = row | (unit << 12);                   // bits 8 and up: the unit's byte offset in the row
  }
  // a chunk's copies in two steps: src_of reads the slots and forms each copy's source
  // address (every slot is read before the first copy goes out: a copy's asm statement is
  // a memory barrier for the compiler, so a read placed after one would wait for LDS on
  // its own); fire(k) then issues copy k, possibly interleaved with other work
  struct Copies {
    int32_t slot[kLoadsHi];                     // -1: masked row, copied from the zero row
  };
  // chunk ci's slots: chunk ci of the segment; SEGS, the chunk's block is ci / 32, whose slots
  // sit in half (ci / 32) % 2 of slot_s
  auto cidx = [](int ci) { return SEGS ? ci & (2 * kMaxSplitRows / kChunk - 1) : ci; };
  auto src_of = [&](int ci) {
    Copies cp;
    const int32_t* srow = slot_s + cidx(ci) * kChunk;
#pragma unroll
    for (int k = 0; k < kLoadsHi; ++k) cp.slot[k] = (k < kLoadsLo || hi) ? srow[lpos[k] & 0xff] : -1;
    return cp;
  };
  auto fire = [&](const Copies& cp, int ci, int k) {
    if (!(k < kLoadsLo || hi)) return;
    const int32_t sl = umode && cp.slot[k] >= 0 ? cp.slot[k] & ((1 << SMLA_UNION_ROW_BITS) - 1) : cp.slot[k];
    if constexpr (BYIDX) {
      dma16_row(rrsrc, (uint32_t)sl, (uint32_t)lpos[k] >> 8, kvbuf[ci % kNBuf] + (k * kS1Waves + w) * 1024);
      return;
    }
    const int unit = lpos[k] >> 12;
    const bool live = sl >= 0;
    const uint32_t slot = live ? (uint32_t)sl : 0u;
    const char* src;
    if constexpr (!kFp8) {
      src = (live ? (const char*)a.kv.rows : (const char*)kZeroRow) + (uint64_t)slot * row_stride32 + unit * 16;
    } else {
      const bool lat = unit < 32;
      const char* plane = live ? (lat ? lat8 : rope16_m32) : (const char*)kZeroRow;
      src = plane + (uint64_t)slot * (lat ? lat8_stride32 : rope16_stride32) + unit * 16;
    }
    dma16(src, kvbuf[ci % kNBuf] + (k * kS1Waves + w) * 1024);
  };
  auto issue = [&](int ci) {
    const Copies cp = src_of(ci);
#pragma unroll
    for (int k = 0; k < kLoadsHi; ++k) fire(cp, ci, k);
  };
  auto no_hook = [](int) {};

  // fp8: chunk ci's rows converted to bf16 rows into staging tile ci % 2, exactly (every e4m3
  // value is a bf16 value; the row scale is applied to the scores and the weights instead).
  // Thread (r, j) = (tid / 16, tid % 16) converts latent units j and 16 + j of row r (16 codes
  // each) into bf16 units 2j, 2j + 1 and 32 + 2j, 33 + 2j (stored at their swizzled positions);
  // lanes j >= 8 write their two units in the other order, so that each 16-lane group of a
  // store covers the 16 bank groups once. Threads 0 .. 255 copy the rotary units (row
  // tid / 8, unit tid % 8: bf16 already). In three parts, so that the loop can place them
  // between MFMAs: 0 reads, 1 and 2 convert and write.
  uint4 su[2], srp;
  auto stage_part = [&](int ci, int part) {
    if constexpr (kFp8) {
      const int r = tid >> 4, j = tid & 15, e = j >> 3, rr = tid >> 3;
      if (part == 0) {
        const char* src = kvbuf[ci % kNBuf];
        su[0] = *(const uint4*)(src + r * kRowBytes + 16 * swz<SMLA_FP8_E4M3>(r, j));
        su[1] = *(const uint4*)(src + r * kRowBytes + 16 * swz<SMLA_FP8_E4M3>(r, 16 + j));
        if (tid < 256) srp = *(const uint4*)(src + rr * kRowBytes + 16 * swz<SMLA_FP8_E4M3>(rr, 32 + (tid & 7)));
      } else {
        char* dst = stg[ci & 1];
        const uint4 u = su[part - 1];
        const int b = 32 * (part - 1), kb = swz_key<SMLA_BF16>(r);
        auto put = [&](int unit, uint32_t w0, uint32_t w1) {
          *(bf16x8*)(dst + r * (kStgBytes / kChunk) + 16 * (unit ^ kb)) = e4m3x8_to_bf16x8(w0, w1);
        };
        put(b + 2 * j + e, e ? u.z : u.x, e ? u.w : u.y);
        put(b + 2 * j + 1 - e, e ? u.x : u.z, e ? u.y : u.w);
        if (part == 2 && tid < 256)
          *(uint4*)(dst + rr * (kStgBytes / kChunk) + 16 * swz<SMLA_BF16>(rr, 64 + (tid & 7))) = srp;
      }
    }
  };
  auto stage = [&](int ci) {
    stage_part(ci, 0);
    stage_part(ci, 1);
    stage_part(ci, 2);
  };
  // the rows the loop reads: bf16, the ring; fp8, the staging tiles
  auto rows_of = [&](int ci) -> const char* { return kFp8 ? stg[ci & 1] : kvbuf[ci % kNBuf]; };

  const Offsets off(x, g, c);
  // P V tiles of chunk ci in iteration ci: fp8, tiles 0 .. kPv0 - 1 while chunk ci + 1 is
  // converted; then (both) tiles kPv0 .. kPvS - 1 with the scores of chunk ci + 1, tiles
  // kPvS .. kPvP - 1 while its weights are formed and published, the rest after the exchange
  constexpr int kPv0 = kFp8 ? kPvF : 0;
  constexpr int kPvS = kFp8 ? kPvF : kPvA;
  constexpr int kPvP = kPvS + kPvPub;
  static_assert(!kFp8 || kPv0 >= 3, "the conversion takes three steps");
  static_assert(kPvPub >= 5 && 16 - kPvP >= 3, "the weights are formed in five steps and taken in three");
  f32x4 oacc[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 sl, sr;

  // Online softmax in base 2 for head h0 + c. Both partners hold the same running max m_run;
  // each forms the weights of its own 16 rows of a chunk and the pair swaps them, so that each
  // lane ends with head c's eight weights (its own rows 16x + 4g + v, then its partner's
  // 16(1 - x) + 4g + v), the A operand of the P V product.
  //   pub(ci, k), k = 0 .. 4, between P V MFMAs of chunk ci - 1: the masked, scaled scores of
  //     the own rows; their weights exp2(s - m_run) when no score of the wave's heads passes
  //     m_run by more than 2^8 (then every weight is at most 2^8), else relative to the head's
  //     own-row max where that one passes it; the weights (times the row scale for fp8) as
  //     bf16 to the exchange, with the reference they are relative to.
  //   absb(k), k = 0 .. 2, after the barrier: the partner's weights and reference. When both
  //     are relative to m_run (nearly every chunk once the first has set the max) the weights
  //     are used as they are; otherwise both sides scale each half by 2^(ref - new max) from
  //     the same bf16 values, so the partners still agree to the bit, and O and the sum are
  //     rescaled (in finish, after the P V MFMAs of chunk ci - 1).
  // Each lane's sum l_own covers its own rows; the partners add theirs at the end.
  float m_run = -INFINITY, l_own = 0.f, l_next = 0.f, mn = -INFINITY, alpha = 1.f;
  float sv[4], pown[4], psum = 0.f, m_use = 0.f, m_par = 0.f;
  int4 lv = make_int4(-1, -1, -1, -1);
  float4 sco = make_float4(1.f, 1.f, 1.f, 1.f);
  uint2 pw = make_uint2(0u, 0u), ppw = make_uint2(0u, 0u);
  int pfast = 1;
  bool wfast = true, up = false;
  bf16x8 pa, pa_next;
  auto pub = [&](int ci, int k) {
    if (k == 0) {
      lv = *(const int4*)(slot_s + cidx(ci) * kChunk + 16 * x + 4 * g);
      if constexpr (kFp8) sco = *(const float4*)(scale_s + cidx(ci) * kChunk + 16 * x + 4 * g);
    } else if (k == 1) {
      const float raw[4] = {kFp8 ? sl[0] * sco.x + sr[0] : sl[0], kFp8 ? sl[1] * sco.y + sr[1] : sl[1],
                            kFp8 ? sl[2] * sco.z + sr[2] : sl[2], kFp8 ? sl[3] * sco.w + sr[3] : sl[3]};
      // a row counts for head h0 + c when its slot is valid and, in union mode, when it names
      // the head's own member
      const int mbit = SMLA_UNION_ROW_BITS + (umode ? (h0 + c) / uH : 0);
      auto ok = [&](int e) { return e >= 0 && (!umode || ((e >> mbit) & 1)); };
      sv[0] = ok(lv.x) ? raw[0] * a.scale_log2 : -INFINITY;
      sv[1] = ok(lv.y) ? raw[1] * a.scale_log2 : -INFINITY;
      sv[2] = ok(lv.z) ? raw[2] * a.scale_log2 : -INFINITY;
      sv[3] = ok(lv.w) ? raw[3] * a.scale_log2 : -INFINITY;
      wfast = !__any(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])) > m_run + 8.0f);
    } else if (k == 2) {
      m_use = m_run;
      if (!wfast) {
        // (also the first rows, with m_run = -inf)
        const float mo = max_rows(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        if (mo > m_run + 8.0f) m_use = mo;
      }
      const float ms = m_use == -INFINITY ? 0.f : m_use;   // no finite score: every weight is 0
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pown[v] = __builtin_amdgcn_exp2f(sv[v] - ms);
        pin(pown[v]);
      }
    } else if (k == 3) {
      psum = (pown[0] + pown[1]) + (pown[2] + pown[3]);
      // the weight that meets row r's values is p * scale(r)
      const float q0 = kFp8 ? pown[0] * sco.x : pown[0], q1 = kFp8 ? pown[1] * sco.y : pown[1];
      const float q2 = kFp8 ? pown[2] * sco.z : pown[2], q3 = kFp8 ? pown[3] * sco.w : pown[3];
      pw = make_uint2(cvt_bf16x2(q0, q1), cvt_bf16x2(q2, q3));
      pin(pw.x); pin(pw.y);
    } else if (k == 4) {
      // the partner took this wave's previous weights before it reached the barrier that this
      // wave passed last, so the slots are free
      px[w][lane] = pw;
      if (g == 0) mx[w][c] = m_use;
      if (lane == 0) fx[w] = wfast ? 1 : 0;
    }
  };
  auto scaled = [](uint32_t wd, float f) {
    return cvt_bf16x2(bf16_to_f32(wd & 0xffffu) * f, bf16_to_f32(wd >> 16) * f);
  };
  auto absb = [&](int k) {
    if (k == 0) {
      ppw = px[w ^ 4][lane];
      m_par = mx[w ^ 4][c];
      pfast = fx[w ^ 4];
    } else if (k == 2) {
      uint2 a0 = pw, a1 = ppw;
      if (wfast && __builtin_amdgcn_readfirstlane(pfast) != 0) {
        mn = m_run;
        up = false;
        l_next = l_own + psum;
      } else {
        // the new running max of head h0 + c; each half's factor 2^(ref - mn) (0 for a half
        // with no finite score yet), O's 2^(m_run - mn)
        mn = fmaxf(m_use, m_par);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float fo = __builtin_amdgcn_exp2f(m_use - ms), fp = __builtin_amdgcn_exp2f(m_par - ms);
        alpha = __builtin_amdgcn_exp2f(m_run - ms);
        up = mn != m_run;
        a0 = make_uint2(scaled(pw.x, fo), scaled(pw.y, fo));
        a1 = make_uint2(scaled(ppw.x, fp), scaled(ppw.y, fp));
        l_next = l_own * alpha + psum * fo;
      }
      pa_next = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
    }
  };
  auto finish = [&]() {
    if (__any(up && m_run != -INFINITY)) {
      // O rows are heads h0 + 4g + v: their factors live in lanes c = 4g + v
      float ah[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) ah[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
      for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) oacc[nt][v] *= ah[v];
    }
    m_run = mn;
    l_own = l_next;
    pa = pa_next;
  };

  // The rows come in segments whose slots are built in LDS. Decode walks one, its split's rows;
  // a split of the segmented form (SEGS, longer than kMaxSplitRows rows) builds its slots a
  // block of kMaxSplitRows rows at a time, the next block while the current one is gathered
  // (page ids and fp8 scales copied ahead), so its ring runs on without a break. The union mode
  // walks its group's union in pieces of kMaxSplitRows entries, each compacted to the entries
  // whose bit names its query; O and the running max and sum carry over from one piece to the
  // next.
  const int nseg = umode ? (len + kMaxSplitRows - 1) / kMaxSplitRows : 1;
  // SEGS: the page ids of block bk (rows r0 + kMaxSplitRows bk ..) into page_s; its slots into
  // half bk % 2 of slot_s (-1 past the split); its fp8 row scales into the same half of scale_s
  const int nblk = (r1 - r0 + kMaxSplitRows - 1) / kMaxSplitRows;
  auto copy_pages = [&](int bk) {
    const int sbn = r0 + bk * kMaxSplitRows;
    const int e0s = sbn >> lp;
    const int n_pg = min((min(sbn + kMaxSplitRows, r1) - 1) >> lp, a.table_width - 1) - e0s + 1;
    for (int k = w; k * 64 < n_pg; k += kS1Waves) {
      const int e = k * 64 + lane;
      dma4(e < n_pg ? (const void*)(trow + e0s + e) : (const void*)kZeroRow, (char*)(page_s + k * 64));
    }
  };
  auto build_block = [&](int bk) {
    const int sbn = r0 + bk * kMaxSplitRows;
    int32_t* const dst = slot_s + (bk & 1) * kMaxSplitRows;
    for (int i = tid; i < kMaxSplitRows; i += kS1Threads) {
      const int p = sbn + i;
      int64_t sl = -1;
      if (p < r1) {
        const int32_t pg = page_s[(p >> lp) - (sbn >> lp)];
        sl = pg < 0 ? -1 : ((int64_t)pg << lp) + (p & ((1 << lp) - 1));
        if (sl >= a.kv.num_slots) sl = -1;
      }
      dst[i] = sl < 0 ? -1 : (int32_t)sl;
    }
  };
  auto copy_scales = [&](int bk, int rows) {
    const int h = (bk & 1) * kMaxSplitRows;
    for (int k = w; k * 64 < rows; k += kS1Waves) {
      const int32_t e = slot_s[h + k * 64 + lane];
      const int32_t sl = umode && e >= 0 ? e & ((1 << SMLA_UNION_ROW_BITS) - 1) : e;
      dma4(sl >= 0 && k * 64 + lane < rows ? (const char*)a.kv.scale + (int64_t)sl * a.kv.scale_stride : (const char*)kZeroRow,
           (char*)(scale_s + h + k * 64));
    }
  };
  for (int seg = 0; seg < nseg; ++seg) {
    const int sb = r0 + seg * kMaxSplitRows;       // first entry (row) of the segment
    if (seg > 0) {
      lds_barrier();                               // every wave is done with the slots and the ring
      const int n_seg = min(kMaxSplitRows, a.max_len - sb);
      for (int k = w; k * 64 < n_seg; k += kS1Waves) {
        const int e = k * 64 + lane;
        dma4(e < n_seg ? (const void*)(trow + sb + e) : (const void*)kZeroRow, (char*)(slot_s + k * 64));
      }
      wait_vmcnt<0>();
      lds_barrier();
    }
    const int nraw = umode ? min(kMaxSplitRows, len - sb) : r1 - r0;
    const int nch_raw = (nraw + kChunk - 1) / kChunk;
    int nrows = nraw;

    // slots of the segment's rows; -1 marks a masked row (past the length, a negative entry or
    // page id, or a slot outside the pool). Union mode keeps the entries whose membership bit
    // names this query (and whose row is in the pool), in union order: a stable block-wide
    // compaction (wave ballots, wave counts through LDS), then -1 past the kept rows up to the
    // chunk boundary.
    if (umode) {
      constexpr int kPer = kMaxSplitRows / kS1Threads;
      uint32_t ent[kPer];
      bool keep[kPer];
      int before[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kS1Threads;
        const uint32_t e = i < nraw ? (uint32_t)slot_s[i] : 0u;
        const uint32_t row = e & ((1u << SMLA_UNION_ROW_BITS) - 1u);
        const uint32_t bits = (e >> (SMLA_UNION_ROW_BITS + m0)) & ((1u << mpw) - 1u);   // this workgroup's members
        ent[k] = row | (bits << SMLA_UNION_ROW_BITS);
        keep[k] = i < nraw && bits != 0u && (int64_t)row < a.kv.num_slots;
        const uint64_t b = __ballot(keep[k]);
        before[k] = __popcll(b & ((1ull << lane) - 1ull));
        if (lane == 0) wcnt[k][w] = __popcll(b);
      }
      lds_barrier();                               // counts published; every entry has been read
      int total = 0, base[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        int pre = 0, tot = 0;
#pragma unroll
        for (int v = 0; v < kS1Waves; ++v) {
          const int n = wcnt[k][v];
          pre += v < w ? n : 0;
          tot += n;
        }
        base[k] = total + pre;
        total += tot;
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (keep[k]) slot_s[base[k] + before[k]] = (int32_t)ent[k];
      nrows = total;
      if (tid < (kChunk - (total & (kChunk - 1))) % kChunk) slot_s[total + tid] = -1;
    } else if (mapped) {
      // positions -> slots exactly as smla_resolve_slots computes them: a position counts when
      // 0 <= pos < the request's context and its page is inside the row with an id >= 0
      constexpr int kPer = kMaxSplitRows / kS1Threads;
      static_assert(kMaxSplitRows % kS1Threads == 0, "rows per thread");
      static_assert(kMaxSplitRows * 4 <= kChunkBytes, "a split's page ids fit one ring slot");
      const int mlp = a.map_log2_page;
      int32_t pos[kPer];
      bool ok[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kS1Threads;
        pos[k] = i < nraw ? slot_s[i] : -1;
        ok[k] = req >= 0 && pos[k] >= 0 && pos[k] < seq && (pos[k] >> mlp) < a.map_pt_width;
      }
      if (!row_in_lds) {
        // the row is longer than a ring slot: each thread copies the page ids of its own
        // positions into ring slot 1 (entry tid + k * kS1Threads) and reads them back
        const int32_t* ptrow = a.map_pt + (int64_t)(req >= 0 ? req : 0) * a.map_pt_stride;
#pragma unroll
        for (int k = 0; k < kPer; ++k)
          dma4(ok[k] ? (const void*)(ptrow + (pos[k] >> mlp)) : (const void*)kZeroRow,
               (char*)(prow_lds + k * kS1Threads + w * 64));
        wait_vmcnt<0>();
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kS1Threads;
        const int32_t page = ok[k] ? prow_lds[row_in_lds ? (pos[k] >> mlp) : i] : -1;
        if (i >= nch_raw * kChunk) continue;
        int64_t sl = -1;
        if (ok[k] && page >= 0) sl = ((int64_t)page << mlp) + (pos[k] & ((1 << mlp) - 1));
        slot_s[i] = (sl < 0 || sl >= a.kv.num_slots) ? -1 : (int32_t)sl;
      }
    } else if (SEGS) {
      build_block(0);                              // (a balanced plan: page size > 1)
    } else {
      for (int i = tid; i < nch_raw * kChunk; i += kS1Threads) {
        int64_t sl = -1;
        if (i < nraw) {
          if (lp == 0) {
            sl = slot_s[i];
          } else {
            const int p = r0 + i;
            const int32_t pg = page_s[(p >> lp) - e0];
            sl = pg < 0 ? -1 : ((int64_t)pg << lp) + (p & ((1 << lp) - 1));
          }
          if (sl >= a.kv.num_slots) sl = -1;
        }
        slot_s[i] = sl < 0 ? -1 : (int32_t)sl;
      }
    }
    lds_barrier();
    if (SEGS && nblk > 1) copy_pages(1);           // page_s is read: block 1's page ids go out
    const int nchunks = (nrows + kChunk - 1) / kChunk;
    if constexpr (kFp8) {
      // the segment's row scales, copied once before its first rows: one 4-byte copy per row
      // into scale_s (masked rows read 0 from the zero row). A per-chunk scale copy inside the
      // loop held each chunk's row gathers up behind it (the fp8 loop took 2.3 instead of 1.3 us
      // per chunk), so the scales go out here, ahead of q and the first chunks, and land before
      // them.
      copy_scales(0, min(nchunks * kChunk, kMaxSplitRows));
    }

    if constexpr (kFp8) {
      // the ring's chunks go out; once chunk 0 (and q and the scales, issued before it) has
      // landed, decode moves q to registers (in its first segment), and chunk 0 is converted
      // into staging tile 0, whose ring slot then takes chunk kNBuf
      for (int ci = 0; ci < kNBuf && ci < nchunks; ++ci) issue(ci);
      wait_chunks_w<kNBuf - 1, kLoadsHi, kLoadsLo>(hi, min(kNBuf - 1, nchunks - 1));
      lds_barrier();
      if (!UNION && seg == 0) {
#pragma unroll
        for (int ks = 0; ks < kQLoads; ++ks) qf[ks] = as_bf16x8(*(const uint4*)(qlds + ks * 1024 + lane * 16));
        lds_barrier();
      }
      if (nchunks == 0) continue;
      stage(0);
      lds_barrier();
      if (kNBuf < nchunks) issue(kNBuf);
    } else {
      if (!UNION && seg == 0) {
        // decode, first segment: chunks 0 and 1 go out; once q (issued in the prologue) has
        // landed every wave moves its quarter to registers, and the slots it held take the
        // next chunks
        for (int ci = 0; ci < 2 && ci < nchunks; ++ci) issue(ci);
        wait_chunks_w<2, kLoadsHi, kLoadsLo>(hi, min(2, nchunks));   // q, issued before them, has landed
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < kQLoads; ++ks) qf[ks] = as_bf16x8(*(const uint4*)(qlds + ks * 1024 + lane * 16));
        lds_barrier();
        for (int ci = 2; ci < kNBuf - 1 && ci < nchunks; ++ci) issue(ci);
      } else {
        for (int ci = 0; ci < kNBuf - 1 && ci < nchunks; ++ci) issue(ci);
      }
      if (nchunks == 0) continue;
      wait_chunks_w<kNBuf - 2, kLoadsHi, kLoadsLo>(hi, min(kNBuf - 2, nchunks - 1));
      lds_barrier();
    }

    // scores and weights of chunk 0
    chunk_step<true, false, kFp8>(rows_of(0), rows_of(0), off, qf, sl, sr, pa, oacc, no_hook);
#pragma unroll
    for (int k = 0; k < 5; ++k) pub(0, k);
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 3; ++k) absb(k);
    finish();

    // iteration ci, in two phases between two barriers: the scores of chunk ci + 1 and its
    // weights (phase A, with the gathers of a later chunk spread over its MFMAs and the
    // weights formed between P V MFMAs of chunk ci), the exchange of weights, then the rest of
    // O += P V over chunk ci with the partner's weights taken in between (phase C).
    // bf16: the barrier at the top publishes chunk ci + 1 and tells that every wave is done
    // with the ring slot of chunk ci - 1, which the iteration refills with chunk ci + kNBuf - 1.
    // fp8: the barrier at the top publishes chunk ci + 1 and frees the staging tile of chunk
    // ci - 1; chunk ci + 1 is converted into it between the first kPv0 P V MFMAs of chunk ci,
    // and after a second barrier its ring slot takes chunk ci + 1 + kNBuf. (The conversion
    // costs about 0.5 us per chunk of LDS and VALU work whether it runs between MFMAs or
    // alone; it replaces a conversion of each MFMA operand, repeated by the four waves that
    // share a row, which was slower.)
    for (int ci = 0; ci + 1 < nchunks; ++ci) {
      if constexpr (kFp8) {
        wait_chunks_w<kNBuf - 1, kLoadsHi, kLoadsLo>(hi, min(kNBuf - 1, nchunks - 2 - ci));
        lds_barrier();
        auto conv = [&](int k) {
          if (k == 0) stage_part(ci + 1, 0);
          else if (k >= kPv0 - 2) stage_part(ci + 1, k - kPv0 + 3);
        };
        chunk_step<false, true, true, decltype((conv)), 0, kPv0>(rows_of(ci), rows_of(ci), off, qf, sl, sr, pa, oacc, conv);
        lds_barrier();
      } else {
        wait_chunks_w<kNBuf - 3, kLoadsHi, kLoadsLo>(hi, min(kNBuf - 3, nchunks - 2 - ci));
        lds_barrier();
      }
      if constexpr (SEGS) {
        // the next block, four chunks into this one: its slots from its page ids (copied a block
        // ago, so older than the copies just waited for); one iteration later, once every
        // thread has built them (barriers between), the block after's page ids and, fp8, the
        // next block's row scales. The next block's gathers start ~30 chunks on, at the end of
        // this block; its half of slot_s last served the block before, finished by then.
        const int bk = ci >> 5;
        if ((ci & 31) == 4 && bk + 1 < nblk) build_block(bk + 1);
        if ((ci & 31) == 5 && bk + 1 < nblk) {
          if (bk + 2 < nblk) copy_pages(bk + 2);
          if constexpr (kFp8) copy_scales(bk + 1, kMaxSplitRows);
        }
      }
      // a copy instruction can wait for room in the compute unit's memory queue: one at a
      // time among the MFMAs, the matrix unit keeps busy meanwhile
      const int cn = kFp8 ? ci + 1 + kNBuf : ci + kNBuf - 1;
      const bool refill = cn < nchunks;
      const Copies cp = src_of(refill ? cn : ci);   // (ci: a valid chunk whose slots go unused)
      auto gathers = [&](int k) {
        if (refill && (k & 3) == 1 && (k >> 2) < kLoadsHi) fire(cp, cn, k >> 2);
      };
      chunk_step<true, (kPvS > kPv0), kFp8, decltype((gathers)), kPv0, kPvS>(rows_of(ci + 1), rows_of(ci), off, qf, sl, sr,
                                                                            pa, oacc, gathers);
      auto pubs = [&](int k) { pub(ci + 1, k); };
      chunk_step<false, true, kFp8, decltype((pubs)), kPvS, kPvP>(rows_of(ci), rows_of(ci), off, qf, sl, sr, pa, oacc, pubs);
      lds_barrier();
      chunk_step<false, true, kFp8, decltype((absb)), kPvP, 16>(rows_of(ci), rows_of(ci), off, qf, sl, sr, pa, oacc, absb);
      finish();
    }
    chunk_step<false, true, kFp8>(rows_of(nchunks - 1), rows_of(nchunks - 1), off, qf, sl, sr, pa, oacc, no_hook);
  }

  // ---- normalise. A token whose rows fit one split is finished here; the others leave
  // their partials for stage 2.
  // head h0 + c, all rows of the split: this wave's rows, then the partner's added in the same
  // order on both sides
  const float lw = sum_rows(l_own);
  if (g == 0) lx[w][c] = lw;
  lds_barrier();
  const float lpar = lx[w ^ 4][c];
  const float l = x == 0 ? lw + lpar : lpar + lw;
  const float lse_c = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  const float inv_c = l > 0.f ? 1.0f / l : 0.0f;
  float inv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) inv[v] = __shfl(inv_c, 4 * g + v, 64);
  if (umode || len <= rps) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = h0 + 4 * g + v;
      if (!writes(hh)) continue;
      uint16_t* ob = (uint16_t*)a.out + (int64_t)tok_of(hh) * a.out_tok_stride + (int64_t)head_of(hh) * a.out_head_stride +
                     256 * x + c;
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) ob[16 * nt] = (uint16_t)cvt_bf16x2(oacc[nt][v] * inv[v], 0.f);
    }
    if (a.lse && x == 0 && g == 0 && writes(h0 + c))
      a.lse[(int64_t)tok_of(h0 + c) * a.lse_tok_stride + head_of(h0 + c)] = lse_c;
    return;
  }
  // (agent-coherent stores: workgroups of this launch may merge them)
  const int64_t part = pbase + s;
  if (x == 0 && g == 0)
    __hip_atomic_store((uint32_t*)a.part_lse + part * kHeads + h0 + c, __float_as_uint(lse_c), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  // bf16 partials in the accumulators' own order, so that one store instruction writes 512
  // contiguous bytes: lane (g, c) of wave (hq, x) stores heads h0 + 4g .. +3 of column
  // 256x + 16nt + c as 8 bytes at ((hq * 2 + x) * 16 + nt) * 64 + lane
  uint64_t* po = (uint64_t*)((uint16_t*)a.part_o + part * (kHeads * kLatent)) + ((hq * 2 + x) * 16 * 64 + lane);
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) {
    const uint64_t v = (uint64_t)cvt_bf16x2(oacc[nt][0] * inv[0], oacc[nt][1] * inv[1]) |
                       ((uint64_t)cvt_bf16x2(oacc[nt][2] * inv[2], oacc[nt][3] * inv[3]) << 32);
    __hip_atomic_store(po + nt * 64, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // (the LDS ring is idle from here on: its first slot holds the merge's LSE staging)
  if (a.sync != nullptr)
    merge_splits(a, t, pbase, tr, kHeads * hbk, hv, min(smax, (len + rps - 1) / rps), wait_ticks, tid,
                 (float*)kvbuf[0]);
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
  int32_t T;
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
  int32_t hblocks;          // packed path: 64-head blocks per token, as in stage 1
  // packed path: the splits were planned on the device from the lengths (balanced_plan, with
  // these arguments), as stage 1 did
  int32_t balanced, min_rows, cus;
};

// Thread = (token, head, 4 consecutive columns); a workgroup of 256 covers two heads. Every
// split's LSE and 16-byte slice are loaded before any arithmetic, so a thread has all its
// splits in flight at once (up to 8 per pass; more splits take further passes with a
// running maximum).
constexpr int kS2Threads = 256;
constexpr int kS2Batch = 8;
__global__ void __launch_bounds__(kS2Threads) decode_stage2(Stage2Args a) {
  // same token -> XCD rule as stage 1, so that the partials come from this XCD's L2
  const int hp_count = (a.H + 1) / 2;
  int t, hp;
  if ((a.T & 7) == 0) {
    const int i = blockIdx.x >> 3;
    t = (blockIdx.x & 7) + 8 * (i / hp_count);
    hp = i % hp_count;
  } else {
    t = blockIdx.x / hp_count;
    hp = blockIdx.x % hp_count;
  }
  const int h = hp * 2 + (threadIdx.x >> 7);
  const int c0 = (threadIdx.x & 127) * 4;
  if (h >= a.H) return;
  int len = a.lens[t];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int nact = min(a.S, (len + a.rows_per_split - 1) / a.rows_per_split);
  const int64_t base = (int64_t)t * a.S;
  float mx = -INFINITY, wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nact; s0 += kS2Batch) {
    float l[kS2Batch];
    float4 o[kS2Batch];
#pragma unroll
    for (int j = 0; j < kS2Batch; ++j) {
      const bool in = s0 + j < nact;
      const int64_t ps = (base + s0 + (in ? j : 0)) * a.H + h;
      l[j] = in ? a.part_lse[ps] : -INFINITY;
      o[j] = in ? *(const float4*)(a.part_o + ps * kLatent + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = mx;
#pragma unroll
    for (int j = 0; j < kS2Batch; ++j) bm = fmaxf(bm, l[j]);
    if (bm == -INFINITY) continue;                   // nothing but empty splits so far
    const float r = expf(mx - bm);                   // 0 on the first non-empty pass
    wsum *= r;
    acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
#pragma unroll
    for (int j = 0; j < kS2Batch; ++j) {
      const float wgt = l[j] == -INFINITY ? 0.f : expf(l[j] - bm);
      wsum += wgt;
      acc.x += wgt * o[j].x; acc.y += wgt * o[j].y; acc.z += wgt * o[j].z; acc.w += wgt * o[j].w;
    }
    mx = bm;
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  if (a.out_f32) {
    float* o = (float*)a.out + (int64_t)t * a.out_tok_stride + (int64_t)h * a.out_head_stride + c0;
    *(float4*)o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint16_t* o = (uint16_t*)a.out + (int64_t)t * a.out_tok_stride + (int64_t)h * a.out_head_stride + c0;
    uint2 v;
    v.x = cvt_bf16x2(acc.x * inv, acc.y * inv);
    v.y = cvt_bf16x2(acc.z * inv, acc.w * inv);
    *(uint2*)o = v;
  }
  if (a.lse && (threadIdx.x & 127) == 0)
    a.lse[(int64_t)t * a.lse_tok_stride + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// Packed bf16 partials of the MFMA path: element (h, col) of one (token, split) sits at
// ((((hq * 2 + x) * 16 + nt) * 4 + g) * 16 + c) * 4 + v with h = 16 hq + 4 g + v and
// col = 256 x + 16 nt + c. Thread = (token, 4 heads 4q .. 4q+3, 4 columns): its 16 values
// are 32 contiguous bytes of every split.
__global__ void __launch_bounds__(kS2Threads) decode_stage2_packed(Stage2Args a) {
  constexpr int kThreadsPerToken = 16 * 128;           // head quads x column quads
  constexpr int kBlocksPerToken = kThreadsPerToken / kS2Threads;
  const int Tv = a.T * a.hblocks;                      // virtual tokens, as in stage 1
  int t, bi;
  if ((Tv & 7) == 0) {
    const int i = blockIdx.x >> 3;
    t = (blockIdx.x & 7) + 8 * (i / kBlocksPerToken);
    bi = i % kBlocksPerToken;
  } else {
    t = blockIdx.x / kBlocksPerToken;
    bi = blockIdx.x % kBlocksPerToken;
  }
  const int j = bi * kS2Threads + threadIdx.x;          // 0 .. 2047
  // consecutive threads take consecutive 32-byte pieces of the packed partial
  const int cq = j & 3, q = (j >> 2) & 15, nt = (j >> 6) & 15, x = j >> 10;   // q = 4 hq + g
  const int hq = q >> 2, g = q & 3;
  const int col0 = 256 * x + 16 * nt + 4 * cq;
  const int hbase = 4 * q;
  const int tr = t % a.T, hbk = t / a.T, hv = min(kHeads, a.H - kHeads * hbk);
  int len = a.lens[tr];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  int rps = a.rows_per_split, smax = a.S;
  int64_t base = (int64_t)t * a.S;
  if (a.balanced) {
    // the plan stage 1 made from the lengths: this token's rows per split and first partial
    __shared__ int sp[2];
    if (threadIdx.x < 64) {
      const BalancedPlan bp = balanced_plan(a.lens, a.T, a.hblocks, a.max_len, a.cus, a.min_rows, threadIdx.x);
      if (threadIdx.x == t) {
        sp[0] = bp.r;
        sp[1] = bp.base;
      }
    }
    __syncthreads();
    rps = sp[0];
    base = sp[1];
    smax = kMaxSplitRows;
  }
  if (len > 0 && len <= rps) return;                   // one split: stage 1 wrote the output
  const int nact = min(smax, (len + rps - 1) / rps);
  const int64_t off = ((((hq * 2 + x) * 16 + nt) * 4 + g) * 16 + 4 * cq) * 4;   // bf16 elements
  const uint16_t* po = (const uint16_t*)a.part_o;
  float mx[4], wsum[4], acc[4][4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    mx[v] = -INFINITY;
    wsum[v] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[v][k] = 0.f;
  }
  for (int s0 = 0; s0 < nact; s0 += kS2Batch) {
    float4 l[kS2Batch];
    uint4 o[kS2Batch][2];
#pragma unroll
    for (int jj = 0; jj < kS2Batch; ++jj) {
      const bool in = s0 + jj < nact;
      const int64_t ps = base + s0 + (in ? jj : 0);
      l[jj] = in ? *(const float4*)(a.part_lse + ps * kHeads + hbase)
                 : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      const uint4* src = (const uint4*)(po + ps * (kHeads * kLatent) + off);
      o[jj][0] = in ? src[0] : make_uint4(0, 0, 0, 0);
      o[jj][1] = in ? src[1] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float bm = mx[v];
#pragma unroll
      for (int jj = 0; jj < kS2Batch; ++jj) bm = fmaxf(bm, ((const float*)&l[jj])[v]);
      if (bm == -INFINITY) continue;
      const float r = expf(mx[v] - bm);
      wsum[v] *= r;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[v][k] *= r;
#pragma unroll
      for (int jj = 0; jj < kS2Batch; ++jj) {
        const float lv = ((const float*)&l[jj])[v];
        const float wgt = lv == -INFINITY ? 0.f : expf(lv - bm);
        wsum[v] += wgt;
        // column 4cq + k of head hbase + v is bf16 element 4k + v of the 16 loaded
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t word = ((const uint32_t*)&o[jj][0])[(4 * k + v) >> 1];
          acc[v][k] += wgt * bf16_to_f32((v & 1) ? (word >> 16) : (word & 0xffffu));
        }
      }
      mx[v] = bm;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (hbase + v >= hv) continue;                     // a head slot past the block's heads
    const int h = kHeads * hbk + hbase + v;
    const float inv = wsum[v] > 0.f ? 1.0f / wsum[v] : 0.f;
    uint16_t* o = (uint16_t*)a.out + (int64_t)tr * a.out_tok_stride + (int64_t)h * a.out_head_stride + col0;
    *(uint2*)o = make_uint2(cvt_bf16x2(acc[v][0] * inv, acc[v][1] * inv), cvt_bf16x2(acc[v][2] * inv, acc[v][3] * inv));
    if (a.lse && nt == 0 && x == 0 && cq == 0)
      a.lse[(int64_t)tr * a.lse_tok_stride + h] = wsum[v] > 0.f ? mx[v] + logf(wsum[v]) : -INFINITY;
  }
}

}  // namespace

namespace {
// Whether stage 1 reads the pool's rows by index through a buffer resource (the BYIDX form):
// a pool of at most 2^32 bytes, a row stride below 2^14 bytes, and for fp8 the rotary part
// right behind the codes in the same row.
bool gathers_by_index(const smla_kv& kv) {
  const bool fp8 = kv.dtype == SMLA_FP8_E4M3;
  const int64_t stride = fp8 ? kv.lat8_stride : kv.row_stride;
  if (stride <= 0 || stride >= (1 << 14) || kv.num_slots > ((int64_t)1 << 32) / stride) return false;
  return !fp8 || ((const char*)kv.rope16 == (const char*)kv.lat8 + 512 && kv.rope16_stride == kv.lat8_stride);
}

template <int KV, bool UNION>
void launch_stage1(dim3 grid, hipStream_t stream, const Stage1Args& a) {
  const bool byidx = gathers_by_index(a.kv);
  if (UNION || !a.balanced) {
    if (byidx)
      hipLaunchKernelGGL((decode_stage1_mfma<KV, UNION, true, false>), grid, dim3(kS1Threads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_stage1_mfma<KV, UNION, false, false>), grid, dim3(kS1Threads), 0, stream, a);
  } else if constexpr (!UNION) {
    if (byidx)
      hipLaunchKernelGGL((decode_stage1_mfma<KV, false, true, true>), grid, dim3(kS1Threads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_stage1_mfma<KV, false, false, true>), grid, dim3(kS1Threads), 0, stream, a);
  }
}
}  // namespace

hipError_t launch_decode(const smla_decode_args& d, const DecodePlan& plan, void* ws, hipStream_t stream,
                         int stages, const smla_page_map* map) {
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
  a.table_width = d.table_width;
  int log2_page = 0;
  while ((1 << log2_page) < d.page_size) ++log2_page;
  a.log2_page = log2_page;
  a.scale_log2 = d.scale * kLog2e;
  a.rows_per_split = plan.rows_per_split;
  a.S = plan.S;
  a.H = d.H;
  a.T = d.T;
  a.part_o = (float*)((char*)ws + plan.sync_bytes);
  a.part_lse = (float*)((char*)ws + plan.sync_bytes + plan.part_o_bytes);
  a.sync = plan.fused ? (uint32_t*)ws : nullptr;
  a.wait_ticks = plan.wait_ticks;
  a.union_G = 0;
  a.hblocks = plan.hblocks;
  a.balanced = plan.balanced;
  a.min_rows = plan.min_rows;
  a.cus = plan.cus;
  a.out = d.out;
  a.out_tok_stride = d.out_tok_stride;
  a.out_head_stride = d.out_head_stride;
  a.lse = d.lse;
  a.lse_tok_stride = d.lse_tok_stride;
  a.mapped = map != nullptr;
  a.map_req = d.lens;                           // a valid [T] array when there is no map
  a.map_pt = nullptr;
  a.map_pt_stride = 0;
  a.map_seq = nullptr;
  a.map_R = a.map_pt_width = a.map_log2_page = 0;
  if (map) {
    a.map_req = map->tok_req;
    a.map_pt = map->page_table;
    a.map_pt_stride = map->pt_stride;
    a.map_seq = map->seq_lens;
    a.map_R = map->R;
    a.map_pt_width = map->pt_width;
    int l = 0;
    while ((1 << l) < map->page_size) ++l;
    a.map_log2_page = l;
  }

  if (!(stages & 1)) {
  } else if (d.q_dtype == SMLA_F32) {
    dim3 grid(plan.S * d.T, (d.H + 15) / 16);
    hipLaunchKernelGGL(decode_stage1_f32, grid, dim3(kThreads), 0, stream, a);
  } else if (d.kv.dtype == SMLA_BF16) {
    launch_stage1<SMLA_BF16, false>(dim3(plan.grid), stream, a);
  } else {
    launch_stage1<SMLA_FP8_E4M3, false>(dim3(plan.grid), stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(stages & 2) || plan.fused) return e;   // fused: stage 1 has merged

  Stage2Args b;
  b.T = d.T;
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
  b.hblocks = plan.hblocks;
  b.balanced = plan.balanced;
  b.min_rows = plan.min_rows;
  b.cus = plan.cus;
  if (d.q_dtype == SMLA_F32)
    hipLaunchKernelGGL(decode_stage2, dim3(d.T * ((d.H + 1) / 2)), dim3(kS2Threads), 0, stream, b);
  else
    hipLaunchKernelGGL(decode_stage2_packed, dim3(d.T * plan.hblocks * (16 * 128 / kS2Threads)), dim3(kS2Threads), 0,
                       stream, b);
  return hipGetLastError();
}

hipError_t launch_stage1_union(const Stage1Args& a, dim3 grid, hipStream_t stream) {
  if (a.kv.dtype == SMLA_BF16)
    launch_stage1<SMLA_BF16, true>(grid, stream, a);
  else
    launch_stage1<SMLA_FP8_E4M3, true>(grid, stream, a);
  return hipGetLastError();
}

namespace {
__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace smla
