// The C ABI of libsmla: host-side argument validation, split and workspace planning,
// error reporting, and dispatch to the kernel launchers. Nothing here touches the GPU
// before every check has passed.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "smla_internal.h"

namespace {

thread_local char g_last_error[512] = "";

smla_status fail(smla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

smla_status ok() {
  g_last_error[0] = '\0';
  return SMLA_OK;
}

smla_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SMLA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

#define CHECK(cond, st, ...)                 \
  do {                                       \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

smla_status check_kv(const smla_kv& kv, const char* fn, bool for_write) {
  CHECK(kv.reserved0 == 0, SMLA_ERR_SHAPE, "%s: kv.reserved0 must be 0", fn);
  CHECK(kv.num_slots > 0, SMLA_ERR_SHAPE, "%s: kv.num_slots must be > 0 (got %lld)", fn, (long long)kv.num_slots);
  // slots travel as int32 through every table of the ABI, so a larger pool has rows no table can name
  CHECK(kv.num_slots <= INT32_MAX, SMLA_ERR_RANGE, "%s: kv.num_slots must be <= 2^31 - 1 (got %lld)", fn,
        (long long)kv.num_slots);
  // the kernels form slot * stride as a 32 x 32 -> 64-bit product, so a row stride must fit 32 bits; the
  // limit is far above any real row (1152 bytes for bf16, 656 for the packed fp8 row)
  CHECK(kv.row_stride < (1ll << 20) && kv.lat8_stride < (1ll << 20) && kv.rope16_stride < (1ll << 20) &&
            kv.scale_stride < (1ll << 20),
        SMLA_ERR_RANGE, "%s: kv row strides must be below 1 MiB", fn);
  if (kv.dtype == SMLA_F32 || kv.dtype == SMLA_BF16) {
    const int64_t row_bytes = kv.dtype == SMLA_F32 ? 4 * SMLA_ROW : 2 * SMLA_ROW;
    CHECK(kv.rows != nullptr, SMLA_ERR_NULL, "%s: kv.rows is NULL", fn);
    CHECK(kv.row_stride >= row_bytes, SMLA_ERR_SHAPE, "%s: kv.row_stride %lld bytes < row size %lld", fn,
          (long long)kv.row_stride, (long long)row_bytes);
    CHECK(aligned(kv.rows, 16) && kv.row_stride % 16 == 0, SMLA_ERR_ALIGN,
          "%s: kv.rows must be 16-byte aligned and kv.row_stride a multiple of 16", fn);
  } else if (kv.dtype == SMLA_FP8_E4M3) {
    CHECK(kv.lat8 && kv.rope16 && kv.scale, SMLA_ERR_NULL, "%s: fp8 kv needs lat8, rope16 and scale", fn);
    CHECK(kv.lat8_stride >= SMLA_LATENT && kv.rope16_stride >= 2 * SMLA_ROPE && kv.scale_stride >= 4,
          SMLA_ERR_SHAPE, "%s: fp8 kv strides too small", fn);
    CHECK(aligned(kv.lat8, 16) && kv.lat8_stride % 16 == 0 && aligned(kv.rope16, 16) &&
              kv.rope16_stride % 16 == 0 && aligned(kv.scale, 4) && kv.scale_stride % 4 == 0,
          SMLA_ERR_ALIGN, "%s: fp8 kv planes misaligned (lat8/rope16: 16 B, scale: 4 B)", fn);
  } else {
    return fail(SMLA_ERR_UNSUPPORTED, "%s: unknown kv dtype %d", fn, kv.dtype);
  }
  (void)for_write;
  return SMLA_OK;
}

// Compute units of the current device (256 on MI355X); the fallback keeps host-only
// callers (workspace queries without a GPU) deterministic.
int32_t device_cus() {
  static int32_t cached[64] = {};           // per device id; a racing first query writes the same value
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

// Ticks of the device's wall clock (s_memrealtime) in `us` microseconds; 100 MHz when the
// attribute is unavailable.
int32_t wall_ticks(int32_t us) {
  static int32_t cached_khz[64] = {};
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return us * 100;
  }
  if (dev >= 0 && dev < 64 && cached_khz[dev] > 0) {
    khz = cached_khz[dev];
  } else if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) {
    (void)hipGetLastError();
    khz = 100000;
  } else if (dev >= 0 && dev < 64) {
    cached_khz[dev] = khz;
  }
  return (int32_t)((int64_t)khz * us / 1000);
}

// Split count and rows per split, from the scalar arguments and the device's compute-unit
// count. A stage-1 workgroup fills a compute unit (its LDS ring), so the default gives
// every compute unit one (token, split) and no second round: floor(CUs / T) splits per
// token, at least enough for the per-split row limit.
// Splits per token when the caller leaves it open: one workgroup per compute unit (CUs / T),
// but no split shorter than min_rows, and none longer than kMaxSplitRows. The floor comes from
// a sweep of split counts for batches 1 .. 128 at top-k 2048: below 128 rows a split's fixed
// cost (first gathers, partial store, merge) outweighs the compute units it adds; at batch 1
// the floor takes the step from 28.6 to 23.2 us (bf16). An fp8 cache's 64-row splits still pay
// while the grid they make is small (batch 1 and 2: 0.2-0.5 us), not beyond (batch 8: 25.4-26
// against 23.4-23.6 us at 128 rows), so check_decode lowers its floor to 64 rows only there.
void plan_splits(int32_t T, int32_t max_len, int32_t requested, int32_t min_rows, int32_t* S_out, int32_t* R_out) {
  const int32_t chunk = smla::kChunk;
  const int32_t max_chunks = (max_len + chunk - 1) / chunk;
  int32_t S;
  if (requested > 0) {
    S = requested;
  } else {
    const int32_t Tq = T > 0 ? T : 1;
    S = device_cus() / Tq;
    const int32_t cap = (max_len + min_rows - 1) / min_rows;
    if (S > cap) S = cap;
    const int32_t need = (max_len + smla::kMaxSplitRows - 1) / smla::kMaxSplitRows;
    if (S < need) S = need;
  }
  if (S > max_chunks) S = max_chunks;
  if (S > 256) S = 256;
  if (S < 1) S = 1;
  int32_t R = (max_len + S - 1) / S;
  R = (R + chunk - 1) / chunk * chunk;
  if (R > smla::kMaxSplitRows) R = smla::kMaxSplitRows;   // a split's slot list lives in LDS
  S = (max_len + R - 1) / R;
  *S_out = S;
  *R_out = R;
}

smla_status check_decode(const smla_decode_args* a, smla::DecodePlan* plan, bool need_ptrs) {
  const char* fn = "smla_sparse_decode";
  CHECK(a != nullptr, SMLA_ERR_NULL, "%s: args is NULL", fn);
  CHECK(a->T >= 0, SMLA_ERR_SHAPE, "%s: T must be >= 0", fn);
  CHECK(a->reserved0 == 0, SMLA_ERR_SHAPE, "%s: reserved0 must be 0", fn);
  const bool bf16 = a->q_dtype == SMLA_BF16;
  if (bf16) {
    CHECK(a->kv.dtype == SMLA_BF16 || a->kv.dtype == SMLA_FP8_E4M3, SMLA_ERR_UNSUPPORTED,
          "%s: bf16 q needs a bf16 or fp8 cache", fn);
    CHECK(a->H >= 1 && a->H <= 128, SMLA_ERR_UNSUPPORTED, "%s: the bf16 path takes 1 <= H <= 128 (got %d)", fn, a->H);
  } else if (a->q_dtype == SMLA_F32) {
    CHECK(a->kv.dtype == SMLA_F32, SMLA_ERR_UNSUPPORTED, "%s: fp32 q needs an fp32 cache", fn);
    CHECK(a->H >= 1 && a->H <= 128, SMLA_ERR_UNSUPPORTED, "%s: the fp32 path takes 1 <= H <= 128", fn);
  } else {
    return fail(SMLA_ERR_UNSUPPORTED, "%s: q_dtype must be SMLA_BF16 or SMLA_F32", fn);
  }
  CHECK(pow2(a->page_size) && a->page_size <= (1 << 20), SMLA_ERR_UNSUPPORTED,
        "%s: page_size must be a power of two in [1, 2^20] (got %d)", fn, a->page_size);
  CHECK(a->table_width >= 1, SMLA_ERR_SHAPE, "%s: table_width must be >= 1", fn);
  CHECK(a->table_stride >= a->table_width, SMLA_ERR_SHAPE, "%s: table_stride < table_width", fn);
  const int64_t max_len = (int64_t)a->table_width * a->page_size;
  CHECK(max_len <= 256 * smla::kMaxSplitRows, SMLA_ERR_RANGE,
        "%s: table_width * page_size exceeds %d (256 splits of %d rows)", fn, 256 * smla::kMaxSplitRows,
        smla::kMaxSplitRows);
  CHECK(a->num_splits >= 0 && a->num_splits <= 256, SMLA_ERR_RANGE, "%s: num_splits must be in [0, 256]", fn);
  CHECK(isfinite(a->scale), SMLA_ERR_SHAPE, "%s: scale must be finite", fn);
  const int64_t qe = bf16 ? 8 : 1;   // q / out row loads are 16 bytes on the bf16 path
  CHECK(a->q_tok_stride >= 0 && a->q_head_stride >= 0 && a->out_tok_stride >= 0 && a->out_head_stride >= 0,
        SMLA_ERR_SHAPE, "%s: strides must be >= 0", fn);
  CHECK(a->q_tok_stride % qe == 0 && a->q_head_stride % qe == 0, SMLA_ERR_ALIGN,
        "%s: bf16 q strides must be multiples of 8 elements", fn);
  const int64_t oe = bf16 ? 8 : 4;
  CHECK(a->out_tok_stride % oe == 0 && a->out_head_stride % oe == 0, SMLA_ERR_ALIGN,
        "%s: out strides must be multiples of 16 bytes", fn);
  if (a->lse) CHECK(a->lse_tok_stride >= a->H, SMLA_ERR_SHAPE, "%s: lse_tok_stride < H", fn);
  smla_status st = check_kv(a->kv, fn, false);
  if (st != SMLA_OK) return st;
  if (need_ptrs && a->T > 0) {
    CHECK(a->q && a->table && a->lens && a->out, SMLA_ERR_NULL, "%s: q, table, lens and out are required", fn);
    CHECK(aligned(a->q, bf16 ? 16 : 4) && aligned(a->out, 16) && aligned(a->table, 4) && aligned(a->lens, 4) &&
              (!a->lse || aligned(a->lse, 4)),
          SMLA_ERR_ALIGN, "%s: q/out must be 16-byte aligned (fp32 q: 4), int32 arrays 4-byte aligned", fn);
  }
  plan->T = a->T;
  plan->H = a->H;
  plan->max_len = (int32_t)max_len;
  // bf16 q: tokens of up to 64 heads are one block, of 65 .. 128 heads two; the splits, the
  // partials and the merge words are per (token, block), each block holding 64 head slots
  plan->hblocks = bf16 ? (a->H + 63) / 64 : 1;
  const int64_t tv = (int64_t)a->T * plan->hblocks;
  CHECK(tv <= (1 << 24), SMLA_ERR_RANGE, "%s: T * ceil(H / 64) must be <= 2^24", fn);
  const int64_t hslots = bf16 ? 64 : a->H;
  int32_t min_rows = !bf16 ? smla::kChunk : 128;
  if (bf16 && a->kv.dtype == SMLA_FP8_E4M3 && tv * ((max_len + 63) / 64) <= device_cus() / 4) min_rows = 64;
  plan_splits((int32_t)tv, (int32_t)max_len, a->num_splits, min_rows, &plan->S, &plan->rows_per_split);
  plan->min_rows = min_rows;
  plan->cus = device_cus();
  // A dense paged decode (page size > 1: contexts of any length) of at most 64 tokens lets the
  // workgroups size the splits from the actual lengths (no host copy of them), so that short
  // and long contexts share the compute units evenly: at most one split per compute unit,
  // a long split walking its rows in segments of kMaxSplitRows. The grid is one workgroup per
  // compute unit.
  plan->balanced = bf16 && a->page_size > 1 && a->num_splits == 0 && tv <= 64 && tv < plan->cus;
  const int64_t items = plan->balanced ? (int64_t)plan->cus : tv * plan->S;
  plan->grid = (int32_t)items;
  // the bf16 path keeps its partial outputs in bf16, the fp32 path in fp32
  plan->part_o_bytes = (size_t)items * hslots * SMLA_LATENT * (bf16 ? 2 : 4);
  plan->part_lse_bytes = (size_t)items * hslots * sizeof(float);
  // bf16 q: the splits of a block merge at the end of stage 1 through a word per block at
  // the head of the workspace; a workgroup waits for its block's other splits (at most
  // 10 us) only when the whole grid is resident at once
  plan->sync_bytes = bf16 ? smla::kSyncBytes : 0;
  plan->fused = bf16 && tv <= smla::kSyncTokens;
  plan->wait_ticks = tv * plan->S <= plan->cus || plan->balanced ? wall_ticks(10) : 0;
  plan->ws_bytes = plan->sync_bytes + (plan->part_o_bytes + plan->part_lse_bytes + 255) / 256 * 256;
  return SMLA_OK;
}

}  // namespace

extern "C" {

const char* smla_status_str(int32_t status) {
  switch (status) {
    case SMLA_OK: return "SMLA_OK";
    case SMLA_ERR_NULL: return "SMLA_ERR_NULL";
    case SMLA_ERR_SHAPE: return "SMLA_ERR_SHAPE";
    case SMLA_ERR_ALIGN: return "SMLA_ERR_ALIGN";
    case SMLA_ERR_UNSUPPORTED: return "SMLA_ERR_UNSUPPORTED";
    case SMLA_ERR_RANGE: return "SMLA_ERR_RANGE";
    case SMLA_ERR_WORKSPACE: return "SMLA_ERR_WORKSPACE";
    case SMLA_ERR_DEVICE: return "SMLA_ERR_DEVICE";
    default: return "SMLA_ERR_UNKNOWN";
  }
}

const char* smla_last_error(void) { return g_last_error; }
int32_t smla_abi_version(void) { return SMLA_ABI_VERSION; }
int32_t smla_sizeof_kv(void) { return (int32_t)sizeof(smla_kv); }
int32_t smla_sizeof_decode_args(void) { return (int32_t)sizeof(smla_decode_args); }
int32_t smla_sizeof_prefill_args(void) { return (int32_t)sizeof(smla_prefill_args); }
int32_t smla_sizeof_page_map(void) { return (int32_t)sizeof(smla_page_map); }

smla_status smla_resolve_slots(const int32_t* idx, int64_t idx_stride, const int32_t* valid,
                               const int32_t* tok_req, int32_t R, const int32_t* page_table,
                               int64_t pt_stride, int32_t pt_width, const int32_t* seq_lens,
                               int32_t page_size, int32_t T, int32_t W, int32_t* slots,
                               int64_t slots_stride, void* stream) {
  const char* fn = "smla_resolve_slots";
  CHECK(T >= 0 && W >= 0, SMLA_ERR_SHAPE, "%s: T and W must be >= 0", fn);
  if (T == 0 || W == 0) return ok();
  CHECK(idx && tok_req && page_table && seq_lens && slots, SMLA_ERR_NULL,
        "%s: idx, tok_req, page_table, seq_lens and slots are required", fn);
  CHECK(R >= 1 && pt_width >= 1, SMLA_ERR_SHAPE, "%s: R and pt_width must be >= 1", fn);
  CHECK(idx_stride >= W && slots_stride >= W && pt_stride >= pt_width, SMLA_ERR_SHAPE,
        "%s: a row stride is smaller than its row", fn);
  CHECK(pow2(page_size) && page_size <= (1 << 20), SMLA_ERR_UNSUPPORTED,
        "%s: page_size must be a power of two in [1, 2^20] (got %d)", fn, page_size);
  CHECK(aligned(idx, 4) && aligned(tok_req, 4) && aligned(page_table, 4) && aligned(seq_lens, 4) &&
            aligned(slots, 4) && (!valid || aligned(valid, 4)),
        SMLA_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  CHECK((int64_t)((W + 255) / 256) * T < (1ll << 31), SMLA_ERR_RANGE, "%s: T * W too large", fn);
  return device_status(smla::launch_resolve(idx, idx_stride, valid, tok_req, R, page_table, pt_stride, pt_width,
                                            seq_lens, page_size, T, W, slots, slots_stride,
                                            (hipStream_t)stream),
                       fn);
}

smla_status smla_sparse_decode_workspace(const smla_decode_args* args, size_t* bytes) {
  CHECK(bytes != nullptr, SMLA_ERR_NULL, "smla_sparse_decode_workspace: bytes is NULL");
  smla::DecodePlan plan;
  smla_status st = check_decode(args, &plan, false);
  if (st != SMLA_OK) return st;
  *bytes = args->T == 0 ? 0 : plan.ws_bytes;
  return ok();
}

smla_status smla_sparse_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "smla_sparse_decode_workspace_init";
  if (workspace_bytes == 0) return ok();
  CHECK(workspace != nullptr, SMLA_ERR_NULL, "%s: workspace is NULL", fn);
  CHECK(aligned(workspace, 256), SMLA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  const size_t n = workspace_bytes < smla::kSyncBytes ? workspace_bytes / 16 * 16 : smla::kSyncBytes;
  return device_status(smla::launch_zero(workspace, n, (hipStream_t)stream), fn);
}

smla_status smla_sparse_decode_splits(const smla_decode_args* args, int32_t* num_splits) {
  CHECK(num_splits != nullptr, SMLA_ERR_NULL, "smla_sparse_decode_splits: num_splits is NULL");
  smla::DecodePlan plan;
  smla_status st = check_decode(args, &plan, false);
  if (st != SMLA_OK) return st;
  *num_splits = plan.S;
  return ok();
}

static smla_status check_page_map(const smla_decode_args* args, const smla_page_map* m) {
  const char* fn = "smla_sparse_decode_topk";
  CHECK(m != nullptr, SMLA_ERR_NULL, "%s: map is NULL", fn);
  CHECK(m->reserved0 == 0, SMLA_ERR_SHAPE, "%s: map->reserved0 must be 0", fn);
  CHECK(args->page_size == 1, SMLA_ERR_UNSUPPORTED, "%s: args->page_size must be 1 (one row per entry)", fn);
  CHECK(args->q_dtype == SMLA_BF16, SMLA_ERR_UNSUPPORTED, "%s: the fused path takes bf16 q", fn);
  CHECK(m->R >= 1 && m->pt_width >= 1 && m->pt_stride >= m->pt_width, SMLA_ERR_SHAPE,
        "%s: map needs R >= 1, pt_width >= 1 and pt_stride >= pt_width", fn);
  CHECK(pow2(m->page_size) && m->page_size <= (1 << 20), SMLA_ERR_UNSUPPORTED,
        "%s: map->page_size must be a power of two in [1, 2^20] (got %d)", fn, m->page_size);
  if (args->T > 0) {
    CHECK(m->tok_req && m->page_table && m->seq_lens, SMLA_ERR_NULL,
          "%s: map->tok_req, page_table and seq_lens are required", fn);
    CHECK(aligned(m->tok_req, 4) && aligned(m->page_table, 4) && aligned(m->seq_lens, 4), SMLA_ERR_ALIGN,
          "%s: map arrays must be 4-byte aligned", fn);
  }
  return SMLA_OK;
}

static smla_status decode_stages(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                                 void* stream, int stages, const smla_page_map* map = nullptr) {
  smla::DecodePlan plan;
  smla_status st = check_decode(args, &plan, true);
  if (st != SMLA_OK) return st;
  if (map) {
    st = check_page_map(args, map);
    if (st != SMLA_OK) return st;
  }
  if (args->T == 0) return ok();
  CHECK(workspace != nullptr && workspace_bytes >= plan.ws_bytes, SMLA_ERR_WORKSPACE,
        "smla_sparse_decode: workspace needs %zu bytes (got %zu)", plan.ws_bytes, workspace_bytes);
  CHECK(aligned(workspace, 256), SMLA_ERR_ALIGN, "smla_sparse_decode: workspace must be 256-byte aligned");
  CHECK((int64_t)args->T * plan.S < (1ll << 31), SMLA_ERR_RANGE, "smla_sparse_decode: T * splits too large");
  return device_status(smla::launch_decode(*args, plan, workspace, (hipStream_t)stream, stages, map),
                       "smla_sparse_decode");
}

}  // extern "C"

// Shared with the allocation-free entry point (noalloc.hip), which owns its workspace.
namespace smla {

smla_status decode_workspace_bytes(const smla_decode_args* args, const smla_page_map* map, size_t* bytes) {
  smla::DecodePlan plan;
  smla_status st = check_decode(args, &plan, true);
  if (st != SMLA_OK) return st;
  if (map) {
    st = check_page_map(args, map);
    if (st != SMLA_OK) return st;
  }
  *bytes = args->T == 0 ? 0 : plan.ws_bytes;
  return ok();
}

smla_status decode_enqueue(const smla_decode_args* args, const smla_page_map* map, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return decode_stages(args, workspace, workspace_bytes, stream, 3, map);
}

smla_status report(smla_status st, const char* msg) { return fail(st, "%s", msg); }

smla_status report_device(hipError_t e, const char* what) { return device_status(e, what); }

}  // namespace smla

extern "C" {

smla_status smla_sparse_decode(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_stages(args, workspace, workspace_bytes, stream, 3);
}

smla_status smla_sparse_decode_stage1(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return decode_stages(args, workspace, workspace_bytes, stream, 1);
}

smla_status smla_sparse_decode_stage2(const smla_decode_args* args, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return decode_stages(args, workspace, workspace_bytes, stream, 2);
}

smla_status smla_sparse_decode_topk(const smla_decode_args* args, const smla_page_map* map, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  CHECK(map != nullptr, SMLA_ERR_NULL, "smla_sparse_decode_topk: map is NULL");
  return decode_stages(args, workspace, workspace_bytes, stream, 3, map);
}

smla_status smla_sparse_decode_topk_stage1(const smla_decode_args* args, const smla_page_map* map,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(map != nullptr, SMLA_ERR_NULL, "smla_sparse_decode_topk_stage1: map is NULL");
  return decode_stages(args, workspace, workspace_bytes, stream, 1, map);
}

smla_status smla_build_group_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                                   int32_t Q, int32_t W, int32_t G, int64_t num_slots,
                                   uint32_t* enc, int64_t enc_stride, int32_t* lens, void* stream) {
  const char* fn = "smla_build_group_union";
  CHECK(Q >= 0 && W >= 1, SMLA_ERR_SHAPE, "%s: Q must be >= 0 and W >= 1", fn);
  CHECK(G == 2 || G == 4 || G == 8, SMLA_ERR_UNSUPPORTED, "%s: G must be 2, 4 or 8 (got %d)", fn, G);
  CHECK((int64_t)G * W <= 16384, SMLA_ERR_RANGE, "%s: G * W must be <= 16384", fn);
  CHECK(num_slots >= 1 && num_slots <= SMLA_UNION_MAX_SLOTS, SMLA_ERR_RANGE,
        "%s: num_slots must be in [1, 2^24 - 2] (got %lld)", fn, (long long)num_slots);
  if (Q == 0) return ok();
  CHECK(slots && enc && lens, SMLA_ERR_NULL, "%s: slots, enc and lens are required", fn);
  CHECK(slots_stride >= W && enc_stride >= (int64_t)G * W, SMLA_ERR_SHAPE, "%s: a row stride is too small", fn);
  CHECK(aligned(slots, 4) && aligned(enc, 4) && aligned(lens, 4) && (!valid || aligned(valid, 4)), SMLA_ERR_ALIGN,
        "%s: arrays must be 4-byte aligned", fn);
  return device_status(smla::launch_union(slots, slots_stride, valid, Q, W, G, num_slots, enc, enc_stride, lens,
                                          device_cus(), (hipStream_t)stream),
                       fn);
}

smla_status smla_grouped_prefill(const smla_prefill_args* a, void* stream) {
  const char* fn = "smla_grouped_prefill";
  CHECK(a != nullptr, SMLA_ERR_NULL, "%s: args is NULL", fn);
  CHECK(a->Q >= 0, SMLA_ERR_SHAPE, "%s: Q must be >= 0", fn);
  CHECK(a->reserved1 == 0, SMLA_ERR_SHAPE, "%s: reserved1 must be 0", fn);
  CHECK((a->G == 2 || a->G == 4 || a->G == 8) && a->G * a->H == 128, SMLA_ERR_UNSUPPORTED,
        "%s: needs G in {2, 4, 8} and G * H == 128 (got G=%d, H=%d)", fn, a->G, a->H);
  CHECK(a->kv.dtype == SMLA_BF16 || a->kv.dtype == SMLA_FP8_E4M3, SMLA_ERR_UNSUPPORTED,
        "%s: the cache must be bf16 or fp8 e4m3", fn);
  CHECK(a->enc_width <= (1 << 24), SMLA_ERR_RANGE, "%s: enc_width must be <= 2^24", fn);
  CHECK(a->enc_width >= 1 && a->enc_stride >= a->enc_width, SMLA_ERR_SHAPE,
        "%s: enc_width must be >= 1 and <= enc_stride", fn);
  CHECK(isfinite(a->scale), SMLA_ERR_SHAPE, "%s: scale must be finite", fn);
  smla_status st = check_kv(a->kv, fn, false);
  if (st != SMLA_OK) return st;
  if (a->Q == 0) return ok();
  CHECK(a->q && a->enc && a->lens && a->out, SMLA_ERR_NULL, "%s: q, enc, lens and out are required", fn);
  CHECK(a->q_tok_stride >= 0 && a->q_head_stride >= 0 && a->out_tok_stride >= 0 && a->out_head_stride >= 0,
        SMLA_ERR_SHAPE, "%s: strides must be >= 0", fn);
  CHECK(aligned(a->q, 16) && a->q_tok_stride % 8 == 0 && a->q_head_stride % 8 == 0, SMLA_ERR_ALIGN,
        "%s: q must be 16-byte aligned with strides multiple of 8 elements", fn);
  CHECK(aligned(a->out, 2) && aligned(a->enc, 4) && aligned(a->lens, 4) && (!a->lse || aligned(a->lse, 4)),
        SMLA_ERR_ALIGN, "%s: misaligned output or index arrays", fn);
  if (a->lse) CHECK(a->lse_tok_stride >= a->H, SMLA_ERR_SHAPE, "%s: lse_tok_stride < H", fn);
  return device_status(smla::launch_prefill(*a, (hipStream_t)stream), fn);
}

smla_status smla_kv_write(const void* src, int32_t src_dtype, int64_t src_stride, const int32_t* slot_mapping,
                          int32_t T, const smla_kv* dst, void* stream) {
  const char* fn = "smla_kv_write";
  CHECK(dst != nullptr, SMLA_ERR_NULL, "%s: dst is NULL", fn);
  CHECK(T >= 0, SMLA_ERR_SHAPE, "%s: T must be >= 0", fn);
  CHECK(src_dtype == SMLA_F32 || src_dtype == SMLA_BF16, SMLA_ERR_UNSUPPORTED, "%s: src must be fp32 or bf16", fn);
  smla_status st = check_kv(*dst, fn, true);
  if (st != SMLA_OK) return st;
  if (T == 0) return ok();
  CHECK(src && slot_mapping, SMLA_ERR_NULL, "%s: src and slot_mapping are required", fn);
  CHECK(src_stride >= SMLA_ROW, SMLA_ERR_SHAPE, "%s: src_stride < 576", fn);
  const int64_t e = src_dtype == SMLA_F32 ? 4 : 8;
  CHECK(aligned(src, 16) && src_stride % e == 0 && aligned(slot_mapping, 4), SMLA_ERR_ALIGN,
        "%s: src must be 16-byte aligned with a row stride of whole 16-byte units", fn);
  return device_status(smla::launch_kv_write(src, src_dtype, src_stride, slot_mapping, T, *dst, (hipStream_t)stream),
                       fn);
}

}  // extern "C"
