// Host-side declarations shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/smla.h"

namespace smla {

// Rows of one stage-1 chunk (the unit of gather, MFMA and online-softmax update).
constexpr int kChunk = 32;
// Most rows one stage-1 split may hold (its slot list is staged in LDS).
constexpr int kMaxSplitRows = 1024;

// Workspace bytes reserved, at offset 0, for the per-token words through which the split
// workgroups of stage 1 share the merge (one 32-bit word per token, 64 bytes apart). The
// region must hold zeros before a workspace is first used; every call returns the words it
// touched to zero, so one buffer serves calls of any shape. Decodes of more tokens than it
// covers merge in a separate stage-2 kernel.
constexpr size_t kSyncBytes = 256 * 1024;
constexpr int32_t kSyncStride = 16;                       // 32-bit words per token
constexpr int32_t kSyncTokens = (int32_t)(kSyncBytes / (4 * kSyncStride));

// Decode plan: everything the launches need, computed from scalar arguments only.
struct DecodePlan {
  int32_t T, H, S;           // tokens, heads, splits
  int32_t hblocks;           // bf16 q: blocks of 64 head slots per token (1 or 2); fp32 q: 1
  int32_t grid;              // stage-1 workgroups
  int32_t balanced;          // the workgroups plan the splits from the lengths (dense paged, <= 64 tokens)
  int32_t min_rows, cus;     // fewest rows per split; compute units of the device
  int32_t rows_per_split;    // multiple of kChunk
  int32_t max_len;           // table_width * page_size
  size_t part_o_bytes;       // [T, S, H, 512]: bf16 (packed order) on the bf16 path, fp32 on the fp32 path
  size_t part_lse_bytes;     // [T, S, H] fp32
  bool fused;                 // bf16 q with T <= kSyncTokens: stage 1 merges the splits itself
  int32_t wait_ticks;        // how long a stage-1 workgroup may wait for its token's other splits (wall-clock ticks)
  size_t sync_bytes;         // kSyncBytes on the bf16 path, else 0 (the partials follow it)
  size_t ws_bytes;
};

hipError_t launch_resolve(const int32_t* idx, int64_t idx_stride, const int32_t* valid,
                          const int32_t* tok_req, int32_t R, const int32_t* page_table,
                          int64_t pt_stride, int32_t pt_width, const int32_t* seq_lens,
                          int32_t page_size, int32_t T, int32_t W, int32_t* slots,
                          int64_t slots_stride, hipStream_t stream);

hipError_t launch_kv_write(const void* src, int32_t src_dtype, int64_t src_stride,
                           const int32_t* slot_mapping, int32_t T, const smla_kv& dst,
                           hipStream_t stream);

// stages: bit 0 = stage 1, bit 1 = stage 2. `map` (nullable): the table holds positions that
// stage 1 resolves through this page map.
hipError_t launch_decode(const smla_decode_args& a, const DecodePlan& plan, void* ws,
                         hipStream_t stream, int stages = 3, const smla_page_map* map = nullptr);

// cus: the device's compute units (the bit-map builder sizes its persistent grid with it)
hipError_t launch_union(const int32_t* slots, int64_t slots_stride, const int32_t* valid,
                        int32_t Q, int32_t W, int32_t G, int64_t num_slots, uint32_t* enc,
                        int64_t enc_stride, int32_t* lens, int32_t cus, hipStream_t stream);

hipError_t launch_prefill(const smla_prefill_args& a, hipStream_t stream);

// Zero-fill bytes / 16 16-byte words at p (a kernel, so it may be captured in a graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// Decode validation and enqueue for callers that own the workspace (abi.hip): the bytes a full
// decode (both stages; map may be NULL) needs, and the enqueue itself. Both validate exactly as
// smla_sparse_decode / smla_sparse_decode_topk do and leave the same messages.
smla_status decode_workspace_bytes(const smla_decode_args* args, const smla_page_map* map, size_t* bytes);
smla_status decode_enqueue(const smla_decode_args* args, const smla_page_map* map, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);
// Record a failure for smla_last_error() and return its status.
smla_status report(smla_status st, const char* msg);
smla_status report_device(hipError_t e, const char* what);

}  // namespace smla
