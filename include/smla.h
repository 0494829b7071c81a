/*
 * libsmla -- sparse Multi-head Latent Attention over a paged latent KV cache, for
 * AMD Instinct MI355X (gfx950). C ABI.
 *
 * One cached token is one 576-wide latent row: 512 latent values followed by 64 rotary
 * values. All heads of a query share that row: a head's score against a row is the
 * softmax scale times the 576-wide dot product of the head's query (absorbed q_nope
 * plus q_rope) with the row, and the value is the row's first 512 columns (vLLM PR
 * 63104, bench_shardq_rank.py: LORA = 512, ROPE = 64, the [..., :LORA] / [..., LORA:]
 * query split and the 512-wide output; "Details": 64 or 128 query heads per KV head).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is device memory owned by the caller (a HIP allocation). The library
 *     never allocates or frees device memory and never synchronises; every call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.
 *     Scratch space comes in through a caller-provided workspace.
 *   - Launch grids depend only on the scalar arguments, never on device data, so a call
 *     may be captured into a HIP graph (IBM Triton paged-attention explainer, section 4
 *     table, "Static Launch Grid").
 *   - Arguments are validated on the host before anything is enqueued. A failed check
 *     returns a status other than SMLA_OK, enqueues nothing, and leaves a message for
 *     smla_last_error() in the calling thread. A failed launch returns SMLA_ERR_DEVICE.
 *   - Data-dependent conditions (a negative or out-of-range index, a padded entry, a
 *     request id or page id out of range) are masked on the device, never trapped.
 *   - bf16 values are passed as their 16-bit patterns; "elements" means units of the
 *     array's own element type.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 4

#define SMLA_LATENT 512          /* latent (value) columns of a cache row */
#define SMLA_ROPE 64             /* rotary columns of a cache row */
#define SMLA_ROW 576             /* SMLA_LATENT + SMLA_ROPE */
#define SMLA_UNION_ROW_BITS 24   /* union entries: row in bits 0..23, member bits above */
/* The union builder supports pools of at most 2^24 - 2 slots; larger pools are
 * refused with SMLA_ERR_RANGE (vLLM PR 63104, "Changes": grouping falls back when the
 * cache has 2^24 - 1 or more KV rows). */
#define SMLA_UNION_MAX_SLOTS ((1 << 24) - 2)
/* Packed fp8 cache row: 512 e4m3 codes, 64 bf16 rotary values, one fp32 scale, padding
 * to a multiple of 16 bytes. */
#define SMLA_FP8_ROW_BYTES 656
#define SMLA_FP8_ROPE_OFFSET 512
#define SMLA_FP8_SCALE_OFFSET 640

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL = 1,        /* a required pointer is NULL */
  SMLA_ERR_SHAPE = 2,       /* a size or stride is negative, zero where it must not be, or inconsistent */
  SMLA_ERR_ALIGN = 3,       /* a pointer or stride breaks the alignment stated for it */
  SMLA_ERR_UNSUPPORTED = 4, /* a dtype, head count, group size or page size the library does not implement */
  SMLA_ERR_RANGE = 5,       /* a size exceeds a documented limit */
  SMLA_ERR_WORKSPACE = 6,   /* the workspace is NULL or smaller than the size the query function gave */
  SMLA_ERR_DEVICE = 7       /* a HIP call or kernel launch failed */
} smla_status;

typedef enum {
  SMLA_F32 = 0,        /* IEEE binary32 */
  SMLA_BF16 = 1,       /* bfloat16 bit patterns */
  SMLA_FP8_E4M3 = 2    /* OCP e4m3 (E4M3FN): bias 7, no infinities, max 448 */
} smla_dtype;

/*
 * One latent KV pool of `num_slots` slots, caller-owned device memory.
 *
 * dtype SMLA_F32 / SMLA_BF16: `rows` points at slot 0's 576 values; `row_stride` is
 *   the distance between consecutive slots in BYTES (a multiple of 16; `rows` 16-byte
 *   aligned).
 * dtype SMLA_FP8_E4M3: three planes, each with its own base and BYTE stride per slot
 *   (`lat8` 512 e4m3 codes, `rope16` 64 bf16 values, `scale` one fp32). The latent
 *   value of column d is decode(lat8[d]) * scale; rotary columns are plain bf16
 *   (the fp8 cache of The Assertion That Changed Everything, "Why This Message Was
 *   Written", with the per-token scale amax / 448). The packed layout puts the three
 *   planes in one row of SMLA_FP8_ROW_BYTES bytes: lat8 = base, rope16 = base + 512,
 *   scale = base + 640, every stride = 656. lat8 and rope16 must be 16-byte aligned
 *   with strides a multiple of 16; scale 4-byte aligned with a stride multiple of 4.
 *   Unused fields are ignored.
 * The decode, prefill and write entry points read or write only the rows their
 * arguments name.
 */
typedef struct {
  int32_t dtype;          /* smla_dtype */
  int32_t reserved0;      /* must be 0 */
  int64_t num_slots;
  void* rows;             int64_t row_stride;     /* SMLA_F32 / SMLA_BF16 */
  void* lat8;             int64_t lat8_stride;    /* SMLA_FP8_E4M3 */
  void* rope16;           int64_t rope16_stride;
  void* scale;            int64_t scale_stride;
} smla_kv;

/* ---------------------------------------------------------------------------------
 * Slot resolution (the virtual block table).
 *
 * slots[t, j] = page_table[r, i / P] * P + i % P, with r = tok_req[t], i = idx[t, j],
 * P = page_size, when j < valid[t] (or valid == NULL), 0 <= r < R, 0 <= i < seq_lens[r],
 * i / P < pt_width and that page id is >= 0; otherwise -1. This is the paged kernels'
 * position-to-slot mapping, which turns request-relative top-k indices into physical
 * slots that a decode kernel can walk as a block table of page size 1 (The Virtual
 * Block Table: Reusing Triton MLA for Sparse Attention on Blackwell GPUs, sections "The
 * Investigation", "The Breakthrough" and "Assumptions and Reasoning", Assumption 1).
 *
 *   idx         int32 [T, W], row stride idx_stride elements (>= W)
 *   valid       int32 [T] or NULL (all W entries count)
 *   tok_req     int32 [T] request of each token
 *   page_table  int32 [R, pt_width], row stride pt_stride elements (>= pt_width)
 *   seq_lens    int32 [R] context length of each request
 *   page_size   power of two, 1 .. 2^20
 *   slots       int32 [T, W] output, row stride slots_stride elements (>= W); may not
 *               alias the inputs
 * T == 0 or W == 0 enqueues nothing and returns SMLA_OK. Bit-exact, no floating point.
 * ------------------------------------------------------------------------------- */
smla_status smla_resolve_slots(const int32_t* idx, int64_t idx_stride, const int32_t* valid,
                               const int32_t* tok_req, int32_t R, const int32_t* page_table,
                               int64_t pt_stride, int32_t pt_width, const int32_t* seq_lens,
                               int32_t page_size, int32_t T, int32_t W, int32_t* slots,
                               int64_t slots_stride, void* stream);

/* ---------------------------------------------------------------------------------
 * Split decode attention over a block table.
 *
 * For every query token t and head h: softmax attention of q[t, h] over the rows its
 * table row names -- page_size 1: the first lens[t] entries of table[t] are slots
 * (entries < 0 skipped: the virtual block table of resolved top-k slots); page_size
 * P > 1: positions 0 .. lens[t]-1 through the page ids in table[t] (the dense paged
 * block table), with page ids < 0 skipped (The Virtual Block Table, "The
 * Breakthrough"). lens[t] is clamped to [0, table_width * page_size].
 *
 * Stage 1 splits each token's rows into num_splits contiguous ranges and computes, per
 * range, a partial output and its log-sum-exp; the ranges are then merged by LSE
 * (IBM Triton paged-attention explainer, section 4 table, "Parallel Tiled Softmax"),
 * all on `stream`, through the workspace. On the bf16 path (T * ceil(H / 64) <= 4096) the merge runs at
 * the end of stage 1: the workgroups of a token take tickets on a counter word in the
 * workspace and share the merge once every partial is written (each waits a bounded
 * time for the others; the last to arrive merges whatever was given up), so one kernel
 * produces out and lse. Otherwise a second kernel (stage 2) merges.
 *
 * Supported combinations:
 *   q_dtype SMLA_BF16, kv dtype SMLA_BF16 or SMLA_FP8_E4M3, 1 <= H <= 128 (bf16 MFMA path:
 *     64 heads fill the four 16-row tiles of a workgroup, so a token of up to 64 heads is one
 *     block of 64 head slots and a token of 65 .. 128 heads two, each block with its own
 *     splits and workgroups; fewer than 64 heads leave slots that compute and are dropped,
 *     which costs MFMA time but no memory traffic);
 *   q_dtype SMLA_F32,  kv dtype SMLA_F32, 1 <= H <= 128 (fp32 path).
 * Outputs: out[t, h, 0..511] in q's dtype; lse[t, h] = natural log of
 * sum_j exp(scale * q.k_j) in fp32, -inf (and out = 0) when a token has no rows.
 * ------------------------------------------------------------------------------- */
typedef struct {
  int32_t T;                 /* query tokens (>= 0) */
  int32_t H;                 /* heads */
  int32_t q_dtype;           /* smla_dtype: SMLA_BF16 or SMLA_F32; `out` has the same dtype */
  int32_t page_size;         /* 1 = table rows are slots; P > 1 (power of two) = page ids */
  const void* q;             int64_t q_tok_stride, q_head_stride;     /* elements; 576 contiguous */
  smla_kv kv;
  const int32_t* table;      int64_t table_stride;                    /* elements, >= table_width */
  int32_t table_width;       /* entries per table row (>= 1) */
  int32_t num_splits;        /* 0 = chosen from the shapes; else 1 .. 256 */
  const int32_t* lens;       /* [T] */
  float scale;               /* softmax scale tau */
  int32_t reserved0;         /* must be 0 */
  void* out;                 int64_t out_tok_stride, out_head_stride; /* elements; 512 contiguous */
  float* lse;                int64_t lse_tok_stride;                  /* NULL = not written; heads contiguous */
} smla_decode_args;

/* Workspace bytes smla_sparse_decode needs for these arguments (a function of the
 * scalar fields only). Validates like smla_sparse_decode, pointers excepted.
 *
 * Workspace contract (bf16 path): its first 256 KiB hold the merge counters and must be
 * zero before the workspace is first used (allocate it zero-filled, or call
 * smla_sparse_decode_workspace_init once); every call returns the counters it used to
 * zero, so a workspace may be reused for calls of any shape, and inside a captured graph.
 * The rest (the partial outputs) needs no initial contents. Calls that share a workspace
 * must not overlap in time (they would share counters and partials). */
smla_status smla_sparse_decode_workspace(const smla_decode_args* args, size_t* bytes);

/* Zero the merge counters of a workspace of `workspace_bytes` bytes (a fill kernel on
 * `stream`, so it may be captured in a graph); needed once per workspace unless it was
 * allocated zero-filled. Errors: SMLA_ERR_NULL (NULL workspace with a nonzero size),
 * SMLA_ERR_ALIGN (not 256-byte aligned), SMLA_ERR_DEVICE (launch failure). */
smla_status smla_sparse_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Number of splits smla_sparse_decode uses for these arguments. Exception: a dense paged
 * decode (page_size > 1) of at most 64 tokens (64 blocks of heads) with num_splits 0 on the
 * bf16 path sizes each token's splits on the device from the actual lengths (rows per split
 * from the launch's total, so that the splits of short and long contexts share the compute
 * units evenly); the count reported is then the one a uniform plan would use. */
smla_status smla_sparse_decode_splits(const smla_decode_args* args, int32_t* num_splits);

/* Enqueue the decode. `workspace` (256-byte aligned) must hold at least the bytes
 * smla_sparse_decode_workspace reports and meet the contract above. */
smla_status smla_sparse_decode(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                               void* stream);

/* The two stages on their own, for callers that time or overlap them. Stage 1 followed
 * by stage 2 (same arguments, same workspace) is exactly smla_sparse_decode. When stage 1
 * merges the splits itself (bf16 path, T * ceil(H / 64) <= 4096) it writes out and lse, and stage 2
 * enqueues nothing; otherwise stage 1 leaves each split's partial output and LSE in the
 * workspace and stage 2 merges them. On the bf16 path a token whose rows fit one split is
 * always written by stage 1 directly. */
smla_status smla_sparse_decode_stage1(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                                      void* stream);
smla_status smla_sparse_decode_stage2(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ---------------------------------------------------------------------------------
 * Sparse decode straight from logical top-k indices: slot resolution fused into the
 * decode.
 *
 * The indexer's top-k entries are request-relative positions; smla_resolve_slots turns
 * them into the page size 1 table that smla_sparse_decode walks (The Virtual Block Table,
 * "The Investigation" and "The Breakthrough"). Here stage 1 resolves each entry itself,
 * through `map`, with exactly the rule of smla_resolve_slots, so the results are bitwise
 * those of smla_resolve_slots followed by smla_sparse_decode with page_size 1, without
 * the intermediate slot array or its kernel.
 *
 *   args       as for smla_sparse_decode, with page_size == 1, `table` = the logical
 *              indices idx [T, table_width] (row stride table_stride) and `lens` = the
 *              valid counts (entries j >= lens[t] are padding). bf16 q only.
 *   map        tok_req [T] (request of each token), page_table [R, pt_width] (row stride
 *              pt_stride, page ids), seq_lens [R], page_size P (power of two, 1 .. 2^20):
 *              position i of request r is slot page_table[r, i / P] * P + i % P when
 *              0 <= r < R, 0 <= i < seq_lens[r], i / P < pt_width and that page id >= 0;
 *              otherwise the entry is masked.
 * The workspace is the one smla_sparse_decode_workspace reports for `args`.
 * smla_sparse_decode_topk_stage1 is stage 1 alone; smla_sparse_decode_stage2 with the
 * same args and workspace finishes it.
 * ------------------------------------------------------------------------------- */
typedef struct {
  const int32_t* tok_req;
  const int32_t* page_table; int64_t pt_stride;   /* elements, >= pt_width */
  const int32_t* seq_lens;
  int32_t R;                 /* requests (>= 1) */
  int32_t pt_width;          /* pages per page-table row (>= 1) */
  int32_t page_size;         /* P */
  int32_t reserved0;         /* must be 0 */
} smla_page_map;

smla_status smla_sparse_decode_topk(const smla_decode_args* args, const smla_page_map* map, void* workspace,
                                    size_t workspace_bytes, void* stream);
smla_status smla_sparse_decode_topk_stage1(const smla_decode_args* args, const smla_page_map* map,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Decode without allocation, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * The full decode of smla_sparse_decode (map == NULL) or of smla_sparse_decode_topk (map
 * != NULL, same page-map contract), with the same validation, kernels, split plan and
 * results, but its workspace is a static device array inside the library instead of caller
 * memory: 34 MiB (35,651,584 bytes) on every GPU the library runs on, held from the
 * library's load until the process ends. The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the caller still passes inputs and outputs.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (two streams, two threads) race and give wrong
 * results; calls on one stream, one after another, are safe. The merge words at the head of
 * the array are cleared by a fill kernel on `stream` at the first call on each device (and
 * every decode leaves them zero); a first call made under graph capture clears them inside
 * the graph and again at the next call that is not captured.
 *
 * Errors: as smla_sparse_decode / smla_sparse_decode_topk; SMLA_ERR_RANGE when the call
 * needs more workspace than the array holds (smla_sparse_decode_workspace reports the need:
 * 64 KiB per (token, 64-head block, split) plus 256 KiB, e.g. 16.6 MiB for batch 32 x 8
 * splits at 64 heads); SMLA_ERR_DEVICE when the device or the array's address cannot be
 * obtained.
 * ------------------------------------------------------------------------------- */
smla_status smla_sparse_decode_noalloc(const smla_decode_args* args, const smla_page_map* map, void* stream);

/* ---------------------------------------------------------------------------------
 * Group top-k union with per-query membership bits.
 *
 * Queries are grouped G at a time in order (group g = queries gG .. min(gG+G, Q)-1; the
 * last group may be short and its missing members own no bits). For each group the
 * output lists, in ascending order, every distinct row r with 0 <= r < num_slots that
 * some member q names among its first valid[q] entries (entries < 0 or >= num_slots
 * ignored), as enc = r | mask << 24 with bit i of mask set when member i names r;
 * lens[g] is the number of such rows. Entries of enc[g] at or past lens[g] are left
 * unspecified. (vLLM PR 63104, "Tests": the union builder's edge cases; "Changes": one
 * union per group of consecutive queries, membership bits keep each query to its own
 * rows, groups may span requests; "Details": the union is gathered once per group.)
 *
 *   slots  int32 [Q, W], row stride slots_stride elements (resolved slots)
 *   valid  int32 [Q] or NULL (all W entries count)
 *   G      2, 4 or 8, with G * W <= 16384
 *   num_slots  1 .. SMLA_UNION_MAX_SLOTS, else SMLA_ERR_RANGE
 *   enc    uint32 [ceil(Q/G), G*W], row stride enc_stride elements (>= G*W)
 *   lens   int32 [ceil(Q/G)]
 * Bit-exact, no floating point. Q == 0 enqueues nothing.
 * ------------------------------------------------------------------------------- */
smla_status smla_build_group_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                                   int32_t Q, int32_t W, int32_t G, int64_t num_slots,
                                   uint32_t* enc, int64_t enc_stride, int32_t* lens, void* stream);

/* ---------------------------------------------------------------------------------
 * Grouped sparse prefill.
 *
 * G consecutive queries with H heads each fill one 128-row tile (G * H == 128): the
 * tile gathers its group's union rows once and row i*H + h (member i, head h) attends,
 * with softmax, only to the union entries whose membership bit i is set (vLLM PR 63104,
 * "Overview": 2, 4 or 8 queries per 128-head row; "Details" and "Changes"). Output rows
 * of members past Q are not written. Same score, value and LSE definitions as decode.
 *
 *   q    bf16 [Q, H, 576] token-major, strides in elements
 *   kv   bf16 pool, or fp8 e4m3 pool (dequantised in the kernel as in decode)
 *   enc, lens  as produced by smla_build_group_union for the same Q and G
 *   out  bf16 [Q, H, 512]; lse fp32 [Q, H] or NULL
 * Supported: G * H == 128 with G in {2, 4, 8} (H = 64, 32, 16); enc_width <= 2^24.
 * On gfx950 64 heads fill four 16-row MFMA tiles: the group's 128 rows run as two
 * workgroups of the decode kernel, each serving 64 / H queries of the group; each walks the
 * group's union in segments, keeps the entries that name one of its queries, and masks each
 * head by its own query's bit. Errors as smla_sparse_decode.
 * ------------------------------------------------------------------------------- */
typedef struct {
  int32_t Q;
  int32_t H;
  int32_t G;
  int32_t enc_width;         /* entries per enc row (G * W); lens[g] is clamped to it */
  const void* q;             int64_t q_tok_stride, q_head_stride;
  smla_kv kv;
  const uint32_t* enc;       int64_t enc_stride;
  const int32_t* lens;
  float scale;
  int32_t reserved1;         /* must be 0 */
  void* out;                 int64_t out_tok_stride, out_head_stride;
  float* lse;                int64_t lse_tok_stride;
} smla_prefill_args;

smla_status smla_grouped_prefill(const smla_prefill_args* args, void* stream);

/* ---------------------------------------------------------------------------------
 * Cache write.
 *
 * Writes row i of src into slot slot_mapping[i] of dst (rows with slot_mapping[i] < 0
 * or >= dst->num_slots are skipped), the write that precedes attention in a decode step
 * (The Assertion That Changed Everything, "The Message": set_kv_buffer, and the fp8
 * cache it refuses). Stored form by dst->dtype:
 *   SMLA_F32  : the float32 value;
 *   SMLA_BF16 : nearest bf16 of the float32 value, ties to even;
 *   SMLA_FP8_E4M3 : amax = max |c| over the 512 latent values, scale = fp32(amax / 448),
 *     code = e4m3(fp32(c / scale)) rounded to nearest, ties to even, saturated at 448
 *     (all codes 0 when scale is 0); rotary values as bf16 (nearest, ties to even);
 *     the scale as fp32.
 *   src        [T, 576] of src_dtype (SMLA_F32 or SMLA_BF16), row stride src_stride
 *              elements, 576 contiguous
 * Duplicate slots within one call race; the stored row is then one of the writers'.
 * ------------------------------------------------------------------------------- */
smla_status smla_kv_write(const void* src, int32_t src_dtype, int64_t src_stride,
                          const int32_t* slot_mapping, int32_t T, const smla_kv* dst, void* stream);

/* ---------------------------------------------------------------------------------
 * Utilities.
 * ------------------------------------------------------------------------------- */
const char* smla_status_str(int32_t status);
/* Message of the last failed call in this thread ("" if none). */
const char* smla_last_error(void);
int32_t smla_abi_version(void);
/* sizeof of the argument structs, for bindings that mirror them. */
int32_t smla_sizeof_kv(void);
int32_t smla_sizeof_decode_args(void);
int32_t smla_sizeof_prefill_args(void);
int32_t smla_sizeof_page_map(void);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
