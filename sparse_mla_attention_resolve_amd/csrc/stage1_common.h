// The stage-1 kernel's pieces (decode, and grouped prefill in union mode): its argument block
// and launch entry for the prefill path, the LDS row layout of a gathered chunk, direct-to-LDS
// copies and their waits, the per-lane MFMA operand offsets and the cross-row reductions.
#pragma once

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

constexpr int kHeads = 64;                  // head slots of a stage-1 workgroup (four 16-row MFMA tiles)

// The stage-1 kernel's argument block (decode, dense paged decode and grouped prefill).
struct Stage1Args {
  const uint16_t* q;
  int64_t q_tok_stride, q_head_stride;
  smla_kv kv;
  const int32_t* table;
  int64_t table_stride;
  const int32_t* lens;
  int32_t max_len;          // table_width * page size
  int32_t table_width;
  int32_t log2_page;
  float scale_log2;         // softmax scale * log2(e): scores are kept in base 2
  int32_t rows_per_split;
  int32_t S;
  int32_t H;
  int32_t T;
  float* part_o;            // fp32 path: [T][S][H][512]; bf16 path: bf16 in the packed order below
  float* part_lse;          // [T][S][H], natural log
  // page map: when `mapped` is set, the (page size 1) table holds request-relative
  // positions, which the kernel resolves through the request's page-table row. map_req is
  // always a valid [T] array (lens when unmapped), so its load needs no branch.
  int32_t mapped;
  const int32_t* map_req;
  const int32_t* map_pt;
  int64_t map_pt_stride;
  const int32_t* map_seq;
  int32_t map_R, map_pt_width, map_log2_page;
  // outputs, written by stage 1 itself for a token whose rows fit one split (bf16 path)
  void* out;
  int64_t out_tok_stride, out_head_stride;
  float* lse;
  int64_t lse_tok_stride;
  // merge inside stage 1 (bf16 q): the per-token words at the head of the workspace
  // (nullptr: stage 2 merges), and how long a workgroup may wait for its token's other
  // splits, in wall-clock ticks (0: never wait)
  uint32_t* sync;
  int32_t wait_ticks;
  // union mode (grouped prefill), when > 0: the G = union_G queries of a group have H heads
  // each (G * H = 128); workgroup t serves 64 / H of them (members m0 .. m0 + 64/H - 1 of
  // group t / (G * H / 64)), its 64 heads being theirs in order. The table row and length are
  // the group's union (entries = row | member bits << 24); the kernel keeps the entries that
  // name one of its members, and each head attends only to its own member's. One split
  // (S = 1); workgroups whose first member is past the last query do nothing.
  int32_t union_G;
  // decode, bf16 q: blocks of 64 heads per token (1, or 2 for H up to 128). Workgroups cover
  // hblocks * T virtual tokens, block-major (virtual token b * T + t is block b of token t),
  // each with 64 head slots; slots past the block's real heads read the block's last head
  // and write nothing. Partials and merge words are per virtual token.
  int32_t hblocks;
  // dense paged decode of at most 64 (virtual) tokens, bf16 q: the workgroups plan the splits
  // themselves from the tokens' lengths (balanced), with at least min_rows rows per split,
  // for a device of `cus` compute units
  int32_t balanced, min_rows, cus;
};

// Launches the stage-1 kernel in union mode (grouped prefill) over `grid` workgroups, for the
// cache format of a.kv (decode.hip).
hipError_t launch_stage1_union(const Stage1Args& a, dim3 grid, hipStream_t stream);

namespace {

// Shared-memory layout of one gathered row: the row's 16-byte units, unit u stored at
// position u ^ key(row), a permutation inside each aligned block of 8 units, so that a 32-row
// chunk is a whole number of 64-lane x 16-byte direct-to-LDS load instructions with no padding.
//   bf16 (1152-byte rows, the rows the MFMA loop reads): key = row & 7 spreads the rows that
//     one operand read touches over the 64 LDS banks: the 16-byte score reads (16 consecutive
//     rows at one unit) and the transposing value reads (rows 4g .. 4g+3 and 16 + 4g .. +3 at
//     two units) are conflict-free (checked with the LDS bank-conflict counter on gfx950);
//   fp8 (640-byte rows of codes and rotary values): key = 0. Only the conversion into bf16
//     rows reads them, 16 consecutive lanes over the 16 units of one row, which meets no
//     conflict in any order.
template <int KV>
struct Lay;
template <>
struct Lay<SMLA_BF16> {
  static constexpr int kUnits = 72;      // 1152-byte row
  static constexpr int kNBuf = 4;        // chunks in the LDS ring
};
template <>
struct Lay<SMLA_FP8_E4M3> {
  static constexpr int kUnits = 40;      // 512 e4m3 codes + 64 bf16 rotary values; scales live apart
  static constexpr int kNBuf = 3;        // chunks in the LDS ring, beside two bf16 staging tiles
};

template <int KV>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (KV == SMLA_BF16) return row & 7;
  else return 0;
}
template <int KV>
__device__ __forceinline__ int swz(int row, int unit) { return unit ^ swz_key<KV>(row); }

// Source of the gathers of masked rows (a row past the list's length, or a -1 entry):
// the LDS tile then holds zeros there, so a zero softmax weight meets finite values.
__device__ const uint4 kZeroRow[72] = {};

// Workgroup barrier that waits for this wave's LDS operations only: the outstanding
// direct-to-LDS gathers of later chunks stay in flight across it.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Materialise v in a register here: the compiler otherwise sinks work whose result is only
// needed later (past the MFMAs it is meant to run between).
template <typename V>
__device__ __forceinline__ void pin(V& v) { __asm__ volatile("" : "+v"(v)); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
// 16-byte direct-to-LDS gather: lane l's 16 bytes at `src` land at lds_wave_base + 16 l.
// Issued through inline assembly on purpose: the compiler does not see a pending LDS
// write, so it adds no wait for it before the LDS reads of other ring slots; the kernel
// orders the ring itself (wait_chunks, then a barrier). M0 is set right here and nothing
// else in these kernels reads it.
__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
}

// A buffer resource over a pool of `n` rows of `stride` bytes (stride < 2^14), read as a
// structured buffer: element i is the row at base + i * stride. The hardware checks i < n
// and reads zeros for any other index; it forms i * stride + offset in 32 bits, so the
// caller uses this form only for pools of at most 2^32 bytes.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 row_rsrc(const void* base, uint32_t stride, uint32_t n) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)p, ((uint32_t)(p >> 32) & 0xffffu) | (stride << 16), n, 0x00020000u};
}

// 16-byte direct-to-LDS copy by row index: lane l's 16 bytes at byte `off` of row `row` of
// the resource land at lds_wave_base + 16 l (zeros when row is outside the pool). One
// instruction for the wave, with no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_row(const u32x4& rsrc, uint32_t row, uint32_t off, char* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  const uint64_t va = (uint64_t)row | ((uint64_t)off << 32);
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 idxen offen lds" ::"v"(va), "s"(rsrc),
                   "s"(m0)
                   : "memory");
}

// 4-byte direct-to-LDS copy: lane l's word at `src` lands at lds_wave_base + 4 l.
__device__ __forceinline__ void dma4(const void* src, char* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base);
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory");
}

// Wait until at most `chunks` chunks of `LOADS` gathers each are still in flight.
template <int MAXC, int LOADS>
__device__ __forceinline__ void wait_chunks(int chunks) {
  if constexpr (MAXC > 0) {
    if (chunks >= MAXC) { wait_vmcnt<MAXC * LOADS>(); return; }
    wait_chunks<MAXC - 1, LOADS>(chunks);
  } else {
    wait_vmcnt<0>();
  }
}

constexpr int kQLoads = 18;                 // 16-byte q pieces per lane: 16 heads x 72 units / 64 lanes
constexpr int kAhead = 4;                   // LDS operand reads kept in flight ahead of the MFMAs

// Max and sum over the four lanes c, 16 + c, 32 + c, 48 + c (the four 16-lane rows of the
// wave): v_permlane16_swap exchanges rows 0 <-> 1 and 2 <-> 3 between its two operands,
// v_permlane32_swap the two halves, so each returned pair holds both partners' values.
__device__ __forceinline__ float max_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wait until at most `chunks` chunks are in flight for this wave, which issues `hi` or `lo`
// copies per chunk (a compile-time count either way; the choice is wave-uniform).
template <int MAXC, int HI, int LO>
__device__ __forceinline__ void wait_chunks_w(bool hi, int chunks) {
  if (hi) wait_chunks<MAXC, HI>(chunks); else wait_chunks<MAXC, LO>(chunks);
}


// Per-lane LDS byte offsets of wave (hq, x)'s operand reads in a chunk of bf16 rows (the same
// for every chunk; fp8 chunks are dequantised into bf16 rows before the loop reads them).
//   ka[m]: score operand A = K[chunk row 16x + c][dims 32ks + 8g .. +7]: unit 4ks + g sits at
//          4(ks ^ (key >> 2)) + (g ^ (key & 3)): base m = ks & 1, plus 64 ks
//   vo[m]: P V operand B = V[the wave's own rows 16x + 4g .. +3, then its partner's rows
//          16(1 - x) + 4g .. +3][column c of tile 16x + nt], two transposed 16-bit reads
//          (j = 0, 1); the group's lane c points at row 16(j ^ x) + 4g + c/4, columns
//          16(16x + nt) + 4(c%4) .. +3: unit 32x + 2nt + (c%4)/2,
//          stored at 32x + 8(nt >> 2) + 2((nt & 3) ^ (key >> 1)) + (((c%4)/2) ^ (key & 1)):
//          base vo[4j + (nt & 3)], plus 128 (nt >> 2)
struct Offsets {
  int ka[2];
  int vo[8];
  __device__ __forceinline__ Offsets(int x, int g, int c) {
    constexpr int kRowBytes = Lay<SMLA_BF16>::kUnits * 16;
    const int row = 16 * x + c, key = swz_key<SMLA_BF16>(row);
    const int kh = (key >> 2) * 64;
    ka[0] = row * kRowBytes + 16 * (g ^ (key & 3)) + kh;
    ka[1] = row * kRowBytes + 16 * (g ^ (key & 3)) - kh;
    const int b = (c & 3) >> 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * (j ^ x) + 4 * g + (c >> 2), k2 = swz_key<SMLA_BF16>(r);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        vo[4 * j + m] = r * kRowBytes + 512 * x + 32 * (m ^ (k2 >> 1)) + 16 * (b ^ (k2 & 1)) + 8 * (c & 1);
    }
  }
};

}  // namespace

}  // namespace smla
