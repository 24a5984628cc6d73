// Allocation-free split-KV batch decode, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// pkc_batch_decode_paged with a plan needs a device workspace for the plan's integer arrays
// and the fp32 partial states of split requests.  Here that workspace is a fixed device array
// of this library, `scratch` (PKC_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends):
// the call uploads a host-built plan into it and runs the same decode and merge kernels on it.
// Nothing is allocated or freed.  Every call on one GPU uses that GPU's array, so calls that
// overlap on one GPU (on different streams, or from different threads) race; calls on one
// stream run in order.  The kernels write every partial state before the merge reads it, and
// the plan arrays are overwritten by each call, so nothing in the array needs clearing.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "api_internal.h"
#include "plan_core.h"

namespace {

constexpr size_t kScratchBytes = PKC_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// The array lives in device memory; in host code its name is only a stand-in for the symbol,
// so host code uses the address hipGetSymbolAddress returns for the current device instead.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's array, looked up once per device.
pkc_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkc::fail(PKC_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkc::fail(PKC_ERR_UNSUPPORTED, "allocation-free decode: device ordinal out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pkc::fail(PKC_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKC_OK;
}

}  // namespace

extern "C" pkc_status pkc_batch_decode_paged_noalloc(
    const pkc_plan_info* plan, const void* plan_host_buf, size_t plan_host_bytes, const void* q,
    const void* k_pool, const void* v_pool, int64_t num_pages, const int32_t* block_table,
    int32_t max_blocks, const int32_t* cache_seqlens, const int32_t* kv_start, int32_t batch,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    pkc_dtype dtype, float sm_scale, void* o, float* lse, void* stream) {
  try {
    pkc::clear_error();
    if (!plan || plan->magic != PKC_PLAN_MAGIC) return pkc::fail(PKC_ERR_INVALID_ARG, "not a plan (bad magic)");
    if (plan->num_levels != 0)
      return pkc::fail(PKC_ERR_PLAN_MISMATCH, "allocation-free decode needs a plan without levels");
    if (!plan_host_buf || plan_host_bytes < (size_t)plan->int_bytes)
      return pkc::fail(PKC_ERR_INVALID_ARG, "plan_host_buf is NULL or smaller than the plan's integer arrays");
    if ((size_t)plan->dev_bytes > kScratchBytes)
      return pkc::fail(PKC_ERR_WORKSPACE_TOO_SMALL,
                       "the plan needs " + std::to_string(plan->dev_bytes) +
                           " bytes of device workspace; the allocation-free call has " +
                           std::to_string(kScratchBytes) + " (use pkc_batch_decode_paged with a workspace)");
    void* ws = nullptr;
    pkc_status st = scratch_address(&ws);
    if (st != PKC_OK) return st;
    pkc_plan_info pl = *plan;
    pl.dev_ws = (uint64_t)(uintptr_t)ws;
    return pkc::decode_run(false, 1.f, 1.f, &pl, q, k_pool, v_pool, num_pages, block_table, max_blocks,
                           cache_seqlens, kv_start, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                           dtype, sm_scale, o, lse, ws, kScratchBytes, stream, plan_host_buf);
  } catch (...) {
    return pkc::fail(PKC_ERR_INTERNAL, "exception in pkc_batch_decode_paged_noalloc");
  }
}
