// Host-side pieces of the C ABI shared between api.cpp and the allocation-free entry point.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pkc.h"

namespace pkc {

// True when host_buf is page-locked host memory the device can read directly.
bool host_buf_is_pinned(const void* host_buf);

// The paged batch decode behind pkc_batch_decode_paged(_fp8): validates every argument, then
// (when plan_upload_src is not NULL) enqueues the copy of the plan's integer arrays from that
// host buffer into dev_ws, then the decode kernel and, with a plan, the merge pass, all on
// `stream`.  Nothing is enqueued when a check fails.
pkc_status decode_run(bool fp8, float k_scale, float v_scale, const pkc_plan_info* plan,
                      const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_blocks, const int32_t* cache_seqlens,
                      const int32_t* kv_start, int32_t batch, int32_t num_qo_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size, pkc_dtype dtype,
                      float sm_scale, void* o, float* lse, void* dev_ws, size_t dev_bytes,
                      void* stream, const void* plan_upload_src);

}  // namespace pkc
