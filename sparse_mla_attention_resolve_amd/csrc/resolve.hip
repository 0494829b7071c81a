// Logical top-k indices + page table -> physical slots (the virtual block table of
// page size 1 that decode walks). The Virtual Block Table: Reusing Triton MLA for Sparse
// Attention on Blackwell GPUs, "The Investigation" (slot formula) and "Assumptions and
// Reasoning", Assumption 1 (page size 1).
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

// One thread per (token, entry); page_size is a power of two, so / and % are shifts. The slot is
// formed in 64 bits: one that does not fit int32 resolves to -1, as a pool cannot hold it.
__global__ void __launch_bounds__(256) resolve_kernel(
    const int32_t* __restrict__ idx, int64_t idx_stride, const int32_t* __restrict__ valid,
    const int32_t* __restrict__ tok_req, int32_t R, const int32_t* __restrict__ page_table,
    int64_t pt_stride, int32_t pt_width, const int32_t* __restrict__ seq_lens, int32_t log2_page,
    int32_t W, int32_t* __restrict__ slots, int64_t slots_stride) {
  const int blocks_per_token = (W + 255) >> 8;
  const int t = blockIdx.x / blocks_per_token;
  const int j = (blockIdx.x % blocks_per_token) * 256 + threadIdx.x;
  if (j >= W) return;
  int32_t out = -1;
  const int32_t r = tok_req[t];
  const int32_t n = valid ? valid[t] : W;
  if (j < n && r >= 0 && r < R) {
    const int32_t i = idx[(int64_t)t * idx_stride + j];
    if (i >= 0 && i < seq_lens[r]) {
      const int32_t page_no = i >> log2_page;
      if (page_no < pt_width) {
        const int32_t page = page_table[(int64_t)r * pt_stride + page_no];
        // a slot past the int32 range (page id * P >= 2^31) names no row any table can hold: masked
        const int64_t s = ((int64_t)page << log2_page) + (i & ((1 << log2_page) - 1));
        if (page >= 0 && s <= INT32_MAX) out = (int32_t)s;
      }
    }
  }
  slots[(int64_t)t * slots_stride + j] = out;
}

hipError_t launch_resolve(const int32_t* idx, int64_t idx_stride, const int32_t* valid,
                          const int32_t* tok_req, int32_t R, const int32_t* page_table,
                          int64_t pt_stride, int32_t pt_width, const int32_t* seq_lens,
                          int32_t page_size, int32_t T, int32_t W, int32_t* slots,
                          int64_t slots_stride, hipStream_t stream) {
  int log2_page = 0;
  while ((1 << log2_page) < page_size) ++log2_page;
  if (T == 0 || W == 0) return hipSuccess;
  dim3 grid((unsigned)(((W + 255) / 256) * (int64_t)T));
  hipLaunchKernelGGL(resolve_kernel, grid, dim3(256), 0, stream, idx, idx_stride, valid, tok_req, R,
                     page_table, pt_stride, pt_width, seq_lens, log2_page, W, slots, slots_stride);
  return hipGetLastError();
}

}  // namespace smla
