// In-place append of the new token's K and V rows to the paged cache (gfx950).
//
// "Paged attention" page (Hugging Face Transformers docs), decode path: the cache is updated in
// place, and the worked example shows where each sequence's next token goes -- logical block
// cache_seqlens[b] / P of the sequence's block-table row, slot cache_seqlens[b] % P (sequence
// 1 of the example, whose 32 cached tokens fill block 0, writes slot 0 of its pre-allocated
// block 1).  After the append the sequence attends over cache_seqlens[b] + 1 tokens.
//
// One workgroup per request: it copies the request's Hkv x D row of K and of V (head_dim
// contiguous, the pool layout [pages, P, Hkv, D]) with 16-byte stores, then one lane writes the
// new length.  A target block that is outside the table row, unallocated (-1) or names a page
// outside the pool is a caller error: nothing is written and the length stays as it was.
#include "device_common.h"
#include "kernels.h"

namespace pkc {

__global__ __launch_bounds__(256) void append_kv_kernel(const AppendParams p) {
  const int b = blockIdx.x;
  const int32_t len = scalar_load(p.seqlens + b);
  const int32_t blk = len >> p.page_shift;
  int32_t page = -1;
  if (len >= 0 && blk < p.max_blocks) page = scalar_load(p.block_table + (int64_t)b * p.max_blocks + blk);
  const bool ok = page >= 0 && page < p.num_pages;
  if (ok) {
    const int64_t row = ((int64_t)page << p.page_shift) + (len & ((1 << p.page_shift) - 1));
    const int64_t n16 = p.row_bytes / 16;   // 16-byte chunks of one token row (all KV heads)
    const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_new) + b * p.row_bytes);
    const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_new) + b * p.row_bytes);
    uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(p.k_pool) + row * p.row_bytes);
    uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(p.v_pool) + row * p.row_bytes);
    for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
  // Every lane has read the old length (scalar load above) before it is overwritten, so the
  // output may alias cache_seqlens.
  __syncthreads();
  if (p.seqlens_out && threadIdx.x == 0) p.seqlens_out[b] = ok ? len + 1 : len;
}

hipError_t launch_append_kv(const AppendParams& p, int32_t batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kv_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Multi-token append (the prefill / append path): new token i of request b goes to position
// cache_seqlens[b] + i, i.e. block (cache_seqlens[b] + i) / P of the request's table row, slot
// (cache_seqlens[b] + i) % P -- the next-token rule above applied to every new token in order.
// A request whose target blocks are not all allocated (outside the row, -1, or outside the
// pool), or whose row range is inconsistent, writes nothing and keeps its length, so every
// sequence stays contiguous.  Workgroup (x, b) first checks all of request b's target blocks
// (strided over its lanes), then copies rows x, x + gridDim.x, ... of the request; workgroup
// (0, b) writes the new length.  Other workgroups of b read cache_seqlens[b] concurrently, so
// the output never aliases it (checked on the host).
__global__ __launch_bounds__(256) void append_kv_ragged_kernel(const AppendRaggedParams p) {
  const int b = blockIdx.y;
  const int64_t len = scalar_load(p.seqlens + b);
  const int64_t lo = scalar_load(p.new_indptr + b), hi = scalar_load(p.new_indptr + b + 1);
  const int64_t n = hi - lo;
  bool bad = len < 0 || lo < 0 || n < 0 || hi > p.total_new || len + n > INT32_MAX;
  if (!bad && n > 0) {
    const int64_t j0 = len >> p.page_shift, j1 = (len + n - 1) >> p.page_shift;
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks;
    bool mine = j1 >= p.max_blocks;
    for (int64_t j = j0 + threadIdx.x; j <= j1 && j < p.max_blocks; j += blockDim.x) {
      const int32_t page = row[j];
      mine = mine || page < 0 || page >= p.num_pages;
    }
    bad = __syncthreads_or(mine ? 1 : 0) != 0;
  }
  if (!bad) {
    const int64_t n16 = p.row_bytes / 16;   // 16-byte chunks of one token row (all KV heads)
    const int32_t mask = (1 << p.page_shift) - 1;
    for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
      const int64_t t = len + i;
      const int32_t page = scalar_load(p.block_table + (int64_t)b * p.max_blocks + (t >> p.page_shift));
      const int64_t dst_row = ((int64_t)page << p.page_shift) + (t & mask);
      const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_new) + (lo + i) * p.row_bytes);
      const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_new) + (lo + i) * p.row_bytes);
      uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(p.k_pool) + dst_row * p.row_bytes);
      uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(p.v_pool) + dst_row * p.row_bytes);
      for (int64_t c = threadIdx.x; c < n16; c += blockDim.x) {
        kd[c] = ks[c];
        vd[c] = vs[c];
      }
    }
  }
  if (p.seqlens_out && blockIdx.x == 0 && threadIdx.x == 0) p.seqlens_out[b] = (int32_t)(bad ? len : len + n);
}

hipError_t launch_append_kv_ragged(const AppendRaggedParams& p, int32_t batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kv_ragged_kernel, dim3(32, batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkc
