// Decode for callers that cannot allocate: the workspace is a static device array of the
// library instead of caller memory. The kernels and the plan are those of smla_sparse_decode and
// smla_sparse_decode_topk; only where the workspace lives differs.
#include <stdio.h>

#include <mutex>

#include "smla_internal.h"

namespace smla {
namespace {

// Largest workspace a call may need: the 256 KiB of merge words, then the split partials
// (64 KiB of bf16 per (token, 64-head block, split)) and their LSEs. 34 MiB holds a launch of
// up to 512 such partials, twice what one pass over the 256 compute units of an MI355X
// produces (batch 32 x 8 splits, batch 64 x 4, ...).
constexpr size_t kScratchBytes = (size_t)34 << 20;

// One copy per GPU, held from the library's load until the process ends. In host code this
// name is a host-side stand-in, not a device address: host code uses the address
// hipGetSymbolAddress reports for the current device (scratch_of), never the name.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};             // scratch's address on each device, once looked up
bool g_zeroed[kMaxDevices] = {};           // its merge words have been cleared by a launched fill

}  // namespace
}  // namespace smla

extern "C" {

smla_status smla_sparse_decode_noalloc(const smla_decode_args* args, const smla_page_map* map, void* stream) {
  using namespace smla;
  size_t need = 0;
  smla_status st = decode_workspace_bytes(args, map, &need);
  if (st != SMLA_OK) return st;
  if (args->T == 0) return SMLA_OK;
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "smla_sparse_decode_noalloc: the call needs %zu bytes of workspace; the static scratch holds %zu",
             need, kScratchBytes);
    return report(SMLA_ERR_RANGE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report_device(e, "smla_sparse_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return report(SMLA_ERR_DEVICE, "smla_sparse_decode_noalloc: device id >= 64");
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing((hipStream_t)stream, &cap);
  if (e != hipSuccess) return report_device(e, "smla_sparse_decode_noalloc: hipStreamIsCapturing");
  void* ptr = nullptr;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
      // once per device, with that device current: each GPU holds its own copy at its own address
      e = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_ptr[dev] = nullptr;
        return report_device(e, "smla_sparse_decode_noalloc: hipGetSymbolAddress(scratch)");
      }
    }
    ptr = g_ptr[dev];
    // The merge words must be zero before their first use; every decode leaves them zero.
    // They are cleared by a fill kernel on the caller's stream at the first call on a device;
    // a first call made under graph capture clears them in the graph and again at the next
    // eager call, since a captured graph may never be launched.
    clear = !g_zeroed[dev];
    if (clear && cap == hipStreamCaptureStatusNone) g_zeroed[dev] = true;
  }
  if (clear) {
    e = launch_zero(ptr, kSyncBytes, (hipStream_t)stream);
    if (e != hipSuccess) return report_device(e, "smla_sparse_decode_noalloc: clearing the merge words");
  }
  return decode_enqueue(args, map, ptr, kScratchBytes, (hipStream_t)stream);
}

}  // extern "C"
