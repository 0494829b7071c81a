// Grouped sparse prefill (vLLM PR 63104, "Overview": 2, 4 or 8 queries share a 128-head row;
// "Details": the union is gathered once with a mask per query; "Changes": groups are views
// of token-major q and the last group may be short).
//
// On gfx950 the 64 heads a workgroup handles fill four 16-row MFMA tiles, so a group's
// 128 rows (G queries x H heads) run as G * H / 64 workgroups of the stage-1 kernel in union
// mode: each serves 64 / H queries of the group, walks the group's union, keeps the entries
// that name one of its queries, and masks each head's scores by its own query's bit. This file
// maps a prefill call onto that kernel's arguments; the kernel is in decode.hip.
#include "stage1_common.h"

namespace smla {

hipError_t launch_prefill(const smla_prefill_args& d, hipStream_t stream) {
  if (d.Q == 0) return hipSuccess;
  Stage1Args a = {};
  a.q = (const uint16_t*)d.q;
  a.q_tok_stride = d.q_tok_stride;
  a.q_head_stride = d.q_head_stride;
  a.kv = d.kv;
  // the table is the groups' union entries (row | member bits << 24), one row per group, and
  // `lens` the unions' lengths: the kernel reads both at the workgroup's group
  a.table = (const int32_t*)d.enc;
  a.table_stride = d.enc_stride;
  a.lens = d.lens;
  a.max_len = d.enc_width;
  a.table_width = d.enc_width;
  a.log2_page = 0;                              // entries are rows (page size 1)
  a.scale_log2 = d.scale * kLog2e;
  // one split per query: a workgroup walks its group's whole union, kMaxSplitRows entries (one
  // segment of slots in LDS) at a time, and writes its queries' outputs itself
  a.rows_per_split = kMaxSplitRows;
  a.S = 1;
  a.H = d.H;
  a.T = d.Q;
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.mapped = 0;
  a.map_req = d.lens;                           // a valid array at the group index (unused)
  a.out = d.out;
  a.out_tok_stride = d.out_tok_stride;
  a.out_head_stride = d.out_head_stride;
  a.lse = d.lse;
  a.lse_tok_stride = d.lse_tok_stride;
  a.sync = nullptr;                             // nothing to merge
  a.wait_ticks = 0;
  a.union_G = d.G;
  a.hblocks = 1;
  a.balanced = 0;
  a.min_rows = kChunk;
  a.cus = 0;
  // 64 / H queries per workgroup, G * H / 64 workgroups per group; a short last group's
  // missing members' workgroups leave at once
  const dim3 grid((unsigned)(((d.Q + d.G - 1) / d.G) * (d.G * d.H / kHeads)));
  return launch_stage1_union(a, grid, stream);
}

}  // namespace smla
