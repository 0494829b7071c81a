// Grouped sparse prefill (vLLM PR 63104, "Overview": 2, 4 or 8 queries share a 128-head row;
// "Details": the union is gathered once with a mask per query; "Changes": groups are views
// of token-major q and the last group may be short).
//
// On gfx950 the 64 heads a workgroup handles fill four 16-row MFMA tiles, so a group's
// 128 rows (G queries x H heads) run as G * H / 64 workgroups of the decode stage-1 kernel in
// union mode: each serves 64 / H queries of the group, walks the group's union, keeps the
// entries that name one of its queries, and masks each head's scores by its own query's bit.
#include "smla_internal.h"

namespace smla {

hipError_t launch_prefill(const smla_prefill_args& d, hipStream_t stream) {
  if (d.Q == 0) return hipSuccess;
  return launch_union_decode(d, stream);
}

}  // namespace smla
