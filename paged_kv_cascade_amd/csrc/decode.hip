// Paged batch-decode / suffix kernel for gfx950: instantiations for fp32, fp16 and bf16 pools
// (the kernel itself is in decode_kernel.h), and the integer debug exports.
#include "decode_kernel.h"

namespace pkc {

hipError_t launch_decode(pkc_dtype dt, int head_dim, int group, int waves, const DecodeParams& p,
                         int grid_x, hipStream_t s) {
  if (grid_x <= 0) return hipSuccess;
  switch (dt) {
    case PKC_F32: return launch_decode_d<F32>(head_dim, group, waves, p, grid_x, s);
    case PKC_F16: return launch_decode_d<F16>(head_dim, group, waves, p, grid_x, s);
    case PKC_BF16: return launch_decode_d<BF16>(head_dim, group, waves, p, grid_x, s);
  }
  return hipErrorInvalidValue;
}

// Debug export: the physical row each token of each request is read from.
__global__ void debug_gather_kernel(const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* seqlens, const int32_t* kv_start,
                                    int32_t page_shift, int64_t num_pages, int32_t* rows_out,
                                    int32_t max_tokens) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= max_tokens) return;
  const int lo = max(kv_start ? kv_start[b] : 0, 0);
  const int hi = min(seqlens[b], max_blocks << page_shift);
  int64_t r = -1;
  if (t >= lo && t < hi) r = token_row(block_table + (int64_t)b * max_blocks, t, page_shift, num_pages);
  rows_out[(int64_t)b * max_tokens + t] = (int32_t)r;
}

hipError_t launch_debug_gather(const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seqlens, const int32_t* kv_start, int32_t batch,
                               int32_t page_shift, int64_t num_pages, int32_t* rows_out,
                               int32_t max_tokens, hipStream_t s) {
  if (batch <= 0 || max_tokens <= 0) return hipSuccess;
  dim3 grid((max_tokens + 255) / 256, batch), block(256);
  hipLaunchKernelGGL(debug_gather_kernel, grid, block, 0, s, block_table, max_blocks, seqlens,
                     kv_start, page_shift, num_pages, rows_out, max_tokens);
  return hipGetLastError();
}

// Debug export: each CTA walks its item list exactly as the attention kernels do.
__global__ void debug_trace_kernel(const int32_t* indptr, const int32_t* items,
                                   int32_t* trace_out, int32_t max_items_per_cta) {
  const int c = blockIdx.x;
  const int lane = threadIdx.x;
  const int beg = indptr[c], end = indptr[c + 1];
  for (int k = 0; k < max_items_per_cta; ++k) {
    const int it = beg + k;
    if (lane < 8)
      trace_out[((int64_t)c * max_items_per_cta + k) * 8 + lane] =
          it < end ? items[8 * (int64_t)it + lane] : -1;
  }
}

hipError_t launch_debug_trace(const int32_t* indptr, const int32_t* items, int32_t ctas,
                              int32_t* trace_out, int32_t max_items_per_cta, hipStream_t s) {
  if (ctas <= 0 || max_items_per_cta <= 0) return hipSuccess;
  hipLaunchKernelGGL(debug_trace_kernel, dim3(ctas), dim3(64), 0, s, indptr, items, trace_out,
                     max_items_per_cta);
  return hipGetLastError();
}

}  // namespace pkc
