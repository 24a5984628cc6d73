// C ABI entry points of libpkc (host side): argument validation, plan copy, kernel launches on
// the caller's stream, optional per-kernel event timing.  See include/pkc.h for the contract.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "api_internal.h"
#include "kernels.h"
#include "plan_core.h"

using pkc::fail;

namespace {

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

pkc_status hip_fail(hipError_t e, const char* what) {
  return fail(PKC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int g_cached_cus[64] = {0};
std::mutex g_mu;

pkc_status device_cus(int32_t* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64 && g_cached_cus[dev] > 0) {
    *cus = g_cached_cus[dev];
    return PKC_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (dev >= 0 && dev < 64) g_cached_cus[dev] = n;
  *cus = n;
  return PKC_OK;
}

// ---- per-kernel timing ring ---------------------------------------------------------------
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::vector<TimedLaunch> g_pending;
std::vector<hipEvent_t> g_free_events;
int64_t g_launches[4] = {0, 0, 0, 0};
double g_ms[4] = {0, 0, 0, 0};

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  // Timing-only events: recording them performs no system-scope fence, so the bracket adds no
  // cache writeback / invalidation between the kernels it measures (the reader synchronizes on
  // the stop event before taking the elapsed time).
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` and, when timing is on, brackets it with events on the same stream.  Not while
// the stream is being captured into a graph: events recorded there would only be recorded by
// the graph's replays, and the reader would wait on them.
template <typename F>
pkc_status timed(int kind, hipStream_t s, const char* what, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_timing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
      std::lock_guard<std::mutex> lk(g_mu);
      a = take_event();
      b = take_event();
      if (a) (void)hipEventRecord(a, s);
    }
  }
  hipError_t e = launch();
  if (e != hipSuccess) return hip_fail(e, what);
  if (a && b) {
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_mu);
    g_pending.push_back({kind, a, b});
  }
  return PKC_OK;
}

bool dtype_ok(pkc_dtype d) { return d == PKC_F32 || d == PKC_F16 || d == PKC_BF16; }

pkc_status check_shapes(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim,
                        int32_t page_size, pkc_dtype dtype, float sm_scale) {
  if (batch < 0) return fail(PKC_ERR_INVALID_ARG, "batch must be >= 0");
  if (hq <= 0 || hkv <= 0 || hq % hkv)
    return fail(PKC_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  const int g = hq / hkv;
  if (!(g == 1 || g == 2 || g == 4 || g == 8))
    return fail(PKC_ERR_UNSUPPORTED, "group size Hq/Hkv must be 1, 2, 4 or 8");
  if (!(head_dim == 64 || head_dim == 128)) return fail(PKC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!pkc::is_pow2(page_size) || page_size > 1024)
    return fail(PKC_ERR_UNSUPPORTED, "page_size must be a power of two in [1, 1024]");
  if (!dtype_ok(dtype)) return fail(PKC_ERR_UNSUPPORTED, "unknown dtype");
  // Kernels address inside one page with 32-bit byte offsets.
  if ((int64_t)page_size * hkv * head_dim * (dtype == PKC_F32 ? 4 : 2) > INT32_MAX)
    return fail(PKC_ERR_UNSUPPORTED, "one page (page_size * num_kv_heads * head_dim elements) must be under 2 GiB");
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(PKC_ERR_INVALID_ARG, "sm_scale must be positive and finite");
  return PKC_OK;
}

pkc_status check_plan(const pkc_plan_info* plan, int32_t batch, int32_t hq, int32_t hkv,
                      int32_t head_dim, int32_t page_size, const void* dev_ws, size_t dev_bytes) {
  if (plan->magic != PKC_PLAN_MAGIC) return fail(PKC_ERR_PLAN_MISMATCH, "not a plan (bad magic)");
  if (plan->batch != batch || plan->num_qo_heads != hq || plan->num_kv_heads != hkv ||
      plan->head_dim != head_dim || plan->page_size != page_size)
    return fail(PKC_ERR_PLAN_MISMATCH, "plan was built for other shapes");
  if (plan->dev_ws == 0 || plan->dev_ws != (uint64_t)(uintptr_t)dev_ws)
    return fail(PKC_ERR_PLAN_MISMATCH, "plan was copied to another device workspace");
  if (dev_bytes < (size_t)plan->dev_bytes)
    return fail(PKC_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than the plan needs");
  return PKC_OK;
}

// A plan built with defer_upload is still only in its page-locked host buffer: enqueue its copy
// into the workspace ahead of a run that does not bring it over itself.
pkc_status upload_if_deferred(const pkc_plan_info* plan, void* dev_ws, hipStream_t s) {
  if (!plan || plan->host_src == 0) return PKC_OK;
  hipError_t e = pkc::launch_plan_upload(reinterpret_cast<const void*>(plan->host_src), dev_ws, plan->int_bytes, s);
  if (e != hipSuccess) return hip_fail(e, "plan upload launch");
  return PKC_OK;
}

template <typename T>
T* at(void* base, int64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

pkc::DecodeParams decode_params(const void* q, const void* k, const void* v, int64_t num_pages,
                                const int32_t* bt, int32_t max_blocks, const int32_t* seqlens,
                                const int32_t* kv_start, int32_t hq, int32_t hkv,
                                int32_t page_size, float sm_scale, void* o, float* lse) {
  pkc::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.num_pages = num_pages;
  p.block_table = bt;
  p.max_blocks = max_blocks;
  p.seqlens = seqlens;
  p.kv_start = kv_start;
  p.hq = hq;
  p.hkv = hkv;
  p.page_size = page_size;
  p.page_shift = log2i(page_size);
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.v_scale = 1.0f;
  p.o = o;
  p.lse = lse;
  return p;
}

// In-kernel contraction of a decode or cascade run: the merge lists, the write-through flags
// and the arrival counters of the plan.
void set_contraction(pkc::DecodeParams* p, const pkc_plan_info* plan, void* ws, int32_t num_levels) {
  p->merge_ptr = at<int32_t>(ws, plan->off_merge_ptr);
  p->merge_rows = at<int32_t>(ws, plan->off_merge_rows);
  p->nl2 = num_levels + 2;
  p->counters = at<uint32_t>(ws, plan->off_counters);
  p->req_flags = at<int32_t>(ws, plan->off_req_flags);
  p->batch = plan->batch;
}

pkc::MergePlanParams merge_params(const pkc_plan_info* plan, void* ws, int l0, int l1, bool skip_wt,
                                  void* o, float* lse) {
  pkc::MergePlanParams m{};
  m.st_o = at<float>(ws, plan->off_state_o);
  m.st_lse = at<float>(ws, plan->off_state_lse);
  m.merge_ptr = at<int32_t>(ws, plan->off_merge_ptr);
  m.merge_rows = at<int32_t>(ws, plan->off_merge_rows);
  m.req_flags = skip_wt ? at<int32_t>(ws, plan->off_req_flags) : nullptr;
  m.nl2 = plan->num_levels + 2;
  m.l0 = l0;
  m.l1 = l1;
  m.batch = plan->batch;
  m.hq = plan->num_qo_heads;
  m.o = o;
  m.lse = lse;
  return m;
}

// Ragged multi-token queries run as a level whose groups are the requests: their pages come
// from a dense block table, and the causal mask needs each group's query range and length.
struct PrefillLevel {
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* qo_indptr;
  const int32_t* kv_lens;
  int32_t causal;
  void* o;      // final output of write-through items
  float* lse;
  const uint8_t* tree_mask = nullptr;   // optional tree masks (causal only)
  const int32_t* mask_indptr = nullptr;
  int32_t mask_bytes = 0;
};

// FP8 pools (fp8 = true): k_scale folds into the softmax scale, v_scale into the state.
// With pf, lv is unused and the groups' pages are the rows of pf->block_table.
pkc_status run_level(const pkc_plan_info* plan, int level, const void* q, const void* k, const void* v,
                     int64_t num_pages, const pkc_level_dev* lv, pkc_dtype dtype, float sm_scale,
                     void* ws, hipStream_t s, bool fp8 = false, float k_scale = 1.f,
                     float v_scale = 1.f, const PrefillLevel* pf = nullptr, bool bring_plan = false) {
  if (!pf && plan->lvl_groups[level] > 0 && (!lv->kv_page_indptr || !lv->kv_page_indices))
    return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(level) + ": NULL page arrays");
  pkc::PrefixParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.num_pages = num_pages;
  if (pf) {
    p.page_indptr = nullptr;
    p.page_indices = pf->block_table;
    p.table_stride = pf->max_blocks;
    p.grp_qo_indptr = pf->qo_indptr;
    p.grp_kv_lens = pf->kv_lens;
    p.o = pf->o;
    p.lse = pf->lse;
    p.tree_mask = pf->tree_mask;
    p.mask_indptr = pf->mask_indptr;
    p.mask_bytes = pf->mask_bytes;
  } else {
    // Only batch prefill passes an output for write-through level items.
    if (plan->lvl_write_through != 0)
      return fail(PKC_ERR_PLAN_MISMATCH, "a plan with level write-through (batch prefill) runs only "
                                         "through pkc_batch_prefill_paged");
    p.page_indptr = lv->kv_page_indptr;
    p.page_indices = lv->kv_page_indices;
    p.num_page_indices = lv->num_page_indices;
  }
  p.hq = plan->num_qo_heads;
  p.hkv = plan->num_kv_heads;
  p.page_size = plan->page_size;
  p.page_shift = log2i(plan->page_size);
  p.scale_log2 = sm_scale * 1.4426950408889634f * (fp8 ? k_scale : 1.f);
  p.v_scale = fp8 ? v_scale : 1.f;
  p.st_o = at<float>(ws, plan->off_state_o);
  p.st_lse = at<float>(ws, plan->off_state_lse);
  p.indptr = at<int32_t>(ws, plan->off_lvl_indptr[level]);
  p.items = at<int32_t>(ws, plan->off_lvl_items[level]);
  if (bring_plan) {
    // This launch reads its items from the deferred plan's host buffer and copies the plan's
    // integer words into the workspace for the launches after it.
    p.plan_host = reinterpret_cast<const int32_t*>(plan->host_src);
    p.plan_dev = static_cast<int32_t*>(ws);
    p.plan_words = (int32_t)(plan->int_bytes / 4);
  }
  const int g = plan->num_qo_heads / plan->num_kv_heads;
  const int streams = plan->lvl_streams;
  if (streams != 1 && streams != 2) return fail(PKC_ERR_PLAN_MISMATCH, "plan has no level stream count");
  if (pf && pf->causal)
    return timed(1, s, "prefix kernel launch", [&] {
      return fp8 ? pkc::launch_prefill_causal_fp8(dtype, plan->head_dim, g, plan->lvl_tile_q[level], streams,
                                                  p, plan->level_ctas, s)
                 : pkc::launch_prefill_causal(dtype, plan->head_dim, g, plan->lvl_tile_q[level], streams, p,
                                              plan->level_ctas, s);
    });
  return timed(1, s, "prefix kernel launch", [&] {
    return fp8 ? pkc::launch_prefix_fp8(dtype, plan->head_dim, g, plan->lvl_tile_q[level], streams, p,
                                        plan->level_ctas, s)
               : pkc::launch_prefix(dtype, plan->head_dim, g, plan->lvl_tile_q[level], streams, p,
                                    plan->level_ctas, s);
  });
}

}  // namespace

// True when host_buf is page-locked host memory the device can read (hipHostMalloc / torch
// pin_memory); the last answer is cached per pointer.
bool pkc::host_buf_is_pinned(const void* host_buf) {
  static thread_local const void* last = nullptr;
  static thread_local bool last_pinned = false;
  if (host_buf == last) return last_pinned;
  hipPointerAttribute_t attr{};
  bool pinned = false;
  if (hipPointerGetAttributes(&attr, host_buf) == hipSuccess) pinned = attr.type == hipMemoryTypeHost;
  (void)hipGetLastError();  // a pageable pointer leaves an error behind; clear it
  last = host_buf;
  last_pinned = pinned;
  return pinned;
}

namespace {

// Checks the parameters and fills #CTA defaults from the current device.  A stage launches
// #CTA x Hkv workgroups.  Decode workgroups are small (4 waves, a few dozen VGPRs each) and
// several fit on a compute unit, so the decode default is about 8 workgroups per compute
// unit and at least one CTA per request, #CTA = max(ceil(8 x CUs / Hkv), batch): a CTA that
// walks two requests pays its start-up and drain twice, which costs more than an extra
// round of workgroups.  A level's default is one workgroup per compute unit,
// #CTA = max(1, floor(CUs / Hkv)): such a grid runs 8-wave workgroups (two tile streams), and
// a decode step's level then leaves half as many chunk states to fold as with two 4-wave
// workgroups per compute unit (the 32K-prefix, batch-128 cascade step: 190 against 201 us;
// with three levels 315 against 345 us).  Long multi-token levels (prefill) run faster with
// more, smaller workgroups and should pass their own #CTA.
// with_streams: also resolve the level stream count (pkc_plan; buffer sizes do not depend on it,
// and host-side sizing of explicit-#CTA parameters then needs no device).
pkc_status resolve_params(const pkc_plan_params* params, pkc::Resolved* r, bool with_streams) {
  pkc_status st = pkc::check_params(params, false, r);
  if (st != PKC_OK) return st;
  if (r->p.num_ctas != 0 && r->p.level_ctas != 0 && (!with_streams || r->p.level_streams != 0))
    return PKC_OK;
  int32_t cus = 0;
  if ((st = device_cus(&cus)) != PKC_OK) return st;
  if (r->p.num_ctas == 0)
    r->p.num_ctas = (int32_t)std::max<int64_t>(
        std::max<int64_t>(1, r->p.batch), pkc::ceil_div(8 * (int64_t)cus, r->p.num_kv_heads));
  if (r->p.level_ctas == 0)
    r->p.level_ctas = (int32_t)std::max<int64_t>(1, (int64_t)cus / r->p.num_kv_heads);
  // A level whose workgroups fit one per compute unit runs them with 8 waves (two tile streams
  // merged at the end of each item), so every SIMD still holds two waves; otherwise 4-wave
  // workgroups, two per compute unit.
  if (with_streams && r->p.level_streams == 0)
    r->p.level_streams = (int64_t)r->p.level_ctas * r->p.num_kv_heads <= cus ? 2 : 1;
  return PKC_OK;
}

pkc_status check_prefix_supported(pkc_dtype dtype, int32_t page_size) {
  if (dtype != PKC_F16 && dtype != PKC_BF16)
    return fail(PKC_ERR_UNSUPPORTED, "the multi-query prefix kernel needs f16 or bf16 queries");
  if (page_size < 4) return fail(PKC_ERR_UNSUPPORTED, "the multi-query prefix kernel needs page_size >= 4");
  return PKC_OK;
}

pkc_status check_fp8(pkc_dtype q_dtype, float k_scale, float v_scale) {
  if (q_dtype != PKC_F16 && q_dtype != PKC_BF16)
    return fail(PKC_ERR_UNSUPPORTED, "FP8 pools take fp16 or bf16 queries");
  if (!(k_scale > 0.f) || !std::isfinite(k_scale) || !(v_scale > 0.f) || !std::isfinite(v_scale))
    return fail(PKC_ERR_INVALID_ARG, "k_scale and v_scale must be positive and finite");
  return PKC_OK;
}

}  // namespace

#define PKC_TRY_BEGIN \
  try {               \
    pkc::clear_error();
#define PKC_TRY_END(name)                                                   \
  }                                                                         \
  catch (...) {                                                             \
    return fail(PKC_ERR_INTERNAL, std::string("exception in ") + (name));   \
  }

extern "C" {

const char* pkc_status_string(pkc_status s) {
  switch (s) {
    case PKC_OK: return "PKC_OK";
    case PKC_ERR_INVALID_ARG: return "PKC_ERR_INVALID_ARG";
    case PKC_ERR_UNSUPPORTED: return "PKC_ERR_UNSUPPORTED";
    case PKC_ERR_WORKSPACE_TOO_SMALL: return "PKC_ERR_WORKSPACE_TOO_SMALL";
    case PKC_ERR_PLAN_MISMATCH: return "PKC_ERR_PLAN_MISMATCH";
    case PKC_ERR_HIP: return "PKC_ERR_HIP";
    case PKC_ERR_INTERNAL: return "PKC_ERR_INTERNAL";
  }
  return "PKC_UNKNOWN_STATUS";
}

const char* pkc_version(void) { return "pkc 0.1 gfx950"; }

void pkc_abi_struct_sizes(size_t* plan_params, size_t* level_host, size_t* level_dev,
                          size_t* plan_info) {
  if (plan_params) *plan_params = sizeof(pkc_plan_params);
  if (level_host) *level_host = sizeof(pkc_level_host);
  if (level_dev) *level_dev = sizeof(pkc_level_dev);
  if (plan_info) *plan_info = sizeof(pkc_plan_info);
}

pkc_status pkc_device_info(int32_t device, int32_t* num_cus, int32_t* wave_size,
                           int64_t* lds_bytes_per_block) {
  PKC_TRY_BEGIN
  int v = 0;
  hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CUs)");
  if (num_cus) *num_cus = v;
  if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeWarpSize, device)) != hipSuccess)
    return hip_fail(e, "hipDeviceGetAttribute(wave size)");
  if (wave_size) *wave_size = v;
  if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, device)) != hipSuccess)
    return hip_fail(e, "hipDeviceGetAttribute(LDS)");
  if (lds_bytes_per_block) *lds_bytes_per_block = v;
  return PKC_OK;
  PKC_TRY_END("pkc_device_info")
}

pkc_status pkc_plan_buffer_sizes(const pkc_plan_params* params, const pkc_level_host* levels,
                                 int32_t num_levels, size_t* host_bytes, size_t* device_bytes) {
  PKC_TRY_BEGIN
  pkc::Resolved r;
  pkc_status st = resolve_params(params, &r, false);
  if (st != PKC_OK) return st;
  if ((st = pkc::check_levels(levels, num_levels, r.p.batch, false)) != PKC_OK) return st;
  pkc::Layout L;
  if ((st = pkc::compute_layout(r, levels, num_levels, &L)) != PKC_OK) return st;
  if (host_bytes) *host_bytes = (size_t)L.int_bytes;
  if (device_bytes) *device_bytes = (size_t)L.dev_bytes;
  return PKC_OK;
  PKC_TRY_END("pkc_plan_buffer_sizes")
}

pkc_status pkc_plan(const pkc_plan_params* params, const int32_t* kv_lens_h,
                    const pkc_level_host* levels_h, int32_t num_levels, void* host_buf,
                    size_t host_bytes, void* dev_ws, size_t dev_bytes, void* stream,
                    pkc_plan_info* out) {
  PKC_TRY_BEGIN
  pkc::Resolved r;
  pkc_status st = resolve_params(params, &r, true);
  if (st != PKC_OK) return st;
  if (!dev_ws || ((uintptr_t)dev_ws & 255)) return fail(PKC_ERR_INVALID_ARG, "dev_ws must be 256-byte aligned");
  if ((st = pkc::build_plan_host(r, kv_lens_h, levels_h, num_levels, host_buf, host_bytes, out)) != PKC_OK)
    return st;
  if (dev_bytes < (size_t)out->dev_bytes)
    return fail(PKC_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than " + std::to_string(out->dev_bytes) + " bytes");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (r.p.defer_upload) {
    // The run calls bring the plan over (the first level kernel of a cascade, else the
    // upload kernel ahead of the run): they read the page-locked buffer directly.
    if (!pkc::host_buf_is_pinned(host_buf))
      return fail(PKC_ERR_INVALID_ARG, "defer_upload needs a page-locked host buffer");
    out->dev_ws = (uint64_t)(uintptr_t)dev_ws;
    out->host_src = (uint64_t)(uintptr_t)host_buf;
    return PKC_OK;
  }
  if (pkc::host_buf_is_pinned(host_buf)) {
    // A kernel on the caller's queue reads the pinned buffer: no copy-engine synchronisation.
    e = pkc::launch_plan_upload(host_buf, dev_ws, out->int_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "plan upload launch");
  } else {
    e = hipMemcpyAsync(dev_ws, host_buf, (size_t)out->int_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  }
  out->dev_ws = (uint64_t)(uintptr_t)dev_ws;
  return PKC_OK;
  PKC_TRY_END("pkc_plan")
}

}  // extern "C"

pkc_status pkc::decode_run(bool fp8, float k_scale, float v_scale, const pkc_plan_info* plan,
                           const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* cache_seqlens, const int32_t* kv_start, int32_t batch,
                           int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, pkc_dtype dtype, float sm_scale, void* o, float* lse,
                           void* dev_ws, size_t dev_bytes, void* stream, const void* plan_upload_src) {
  pkc_status st = check_shapes(batch, num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sm_scale);
  if (st != PKC_OK) return st;
  if (fp8 && (st = check_fp8(dtype, k_scale, v_scale)) != PKC_OK) return st;
  if (batch == 0) return PKC_OK;
  if (!q || !k_pool || !v_pool || !block_table || !o || !lse)
    return fail(PKC_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!plan && !cache_seqlens) return fail(PKC_ERR_INVALID_ARG, "cache_seqlens is NULL");
  if (num_pages < 1 || max_blocks < 0)
    return fail(PKC_ERR_INVALID_ARG, "num_pages must be >= 1 (masked lanes read row 0 of page 0) and max_blocks >= 0");
  if ((int64_t)max_blocks * page_size > INT32_MAX)
    return fail(PKC_ERR_INVALID_ARG, "max_blocks * page_size exceeds int32");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  pkc::DecodeParams p = decode_params(q, k_pool, v_pool, num_pages, block_table, max_blocks,
                                      cache_seqlens, kv_start, num_qo_heads, num_kv_heads,
                                      page_size, sm_scale, o, lse);
  if (fp8) {
    p.scale_log2 *= k_scale;
    p.v_scale = v_scale;
  }
  const int g = num_qo_heads / num_kv_heads;
  int grid_x = batch;
  if (plan) {
    if ((st = check_plan(plan, batch, num_qo_heads, num_kv_heads, head_dim, page_size, dev_ws, dev_bytes)) != PKC_OK)
      return st;
    if (plan->num_levels != 0) return fail(PKC_ERR_PLAN_MISMATCH, "batch decode needs a plan without levels");
    p.st_o = at<float>(dev_ws, plan->off_state_o);
    p.st_lse = at<float>(dev_ws, plan->off_state_lse);
    p.indptr = at<int32_t>(dev_ws, plan->off_dec_indptr);
    p.items = at<int32_t>(dev_ws, plan->off_dec_items);
    if (plan->dec_contraction == 1) set_contraction(&p, plan, dev_ws, 0);
    grid_x = plan->num_ctas;
    if (!plan_upload_src && plan->host_src) plan_upload_src = reinterpret_cast<const void*>(plan->host_src);
    if (plan_upload_src) {
      // Every check has passed: copy the plan's integer arrays from the host buffer into the
      // workspace on the same stream, ahead of the kernels that read them.
      hipError_t e = pkc::host_buf_is_pinned(plan_upload_src)
                         ? pkc::launch_plan_upload(plan_upload_src, dev_ws, plan->int_bytes, s)
                         : hipMemcpyAsync(dev_ws, plan_upload_src, (size_t)plan->int_bytes,
                                          hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "plan upload");
    }
  }
  const int waves = plan ? plan->dec_waves : 4;
  if ((st = timed(0, s, "decode kernel launch", [&] {
         return fp8 ? pkc::launch_decode_fp8(dtype, head_dim, g, waves, p, grid_x, s)
                    : pkc::launch_decode(dtype, head_dim, g, waves, p, grid_x, s);
       })) != PKC_OK)
    return st;
  if (plan && plan->dec_contraction != 1) {
    // Always enqueued (it skips the requests flagged as written through), so the launches of a
    // run do not depend on the plan's lengths.
    pkc::MergePlanParams m = merge_params(plan, dev_ws, 0, 1, true, o, lse);
    if ((st = timed(2, s, "merge kernel launch", [&] { return pkc::launch_merge_plan(dtype, head_dim, m, s); })) != PKC_OK)
      return st;
  }
  return PKC_OK;
}

extern "C" {

pkc_status pkc_batch_decode_paged(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                  const void* v_pool, int64_t num_pages,
                                  const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* cache_seqlens, const int32_t* kv_start,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t page_size, pkc_dtype dtype,
                                  float sm_scale, void* o, float* lse, void* dev_ws,
                                  size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return pkc::decode_run(false, 1.f, 1.f, plan, q, k_pool, v_pool, num_pages, block_table, max_blocks,
                         cache_seqlens, kv_start, batch, num_qo_heads, num_kv_heads, head_dim,
                         page_size, dtype, sm_scale, o, lse, dev_ws, dev_bytes, stream, nullptr);
  PKC_TRY_END("pkc_batch_decode_paged")
}

pkc_status pkc_batch_decode_paged_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                      const void* v_pool, float k_scale, float v_scale,
                                      int64_t num_pages, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* cache_seqlens,
                                      const int32_t* kv_start, int32_t batch,
                                      int32_t num_qo_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                      float sm_scale, void* o, float* lse, void* dev_ws,
                                      size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return pkc::decode_run(true, k_scale, v_scale, plan, q, k_pool, v_pool, num_pages, block_table,
                         max_blocks, cache_seqlens, kv_start, batch, num_qo_heads, num_kv_heads,
                         head_dim, page_size, q_dtype, sm_scale, o, lse, dev_ws, dev_bytes, stream,
                         nullptr);
  PKC_TRY_END("pkc_batch_decode_paged_fp8")
}

static pkc_status prefix_impl(bool fp8, float k_scale, float v_scale, const pkc_plan_info* plan,
                              int32_t level, const void* q, const void* k_pool, const void* v_pool,
                              int64_t num_pages, const pkc_level_dev* level_dev, int32_t batch,
                              int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, pkc_dtype dtype, float sm_scale, void* o_state,
                              pkc_dtype o_dtype, float* lse_state, void* dev_ws, size_t dev_bytes,
                              void* stream) {
  pkc_status st = check_shapes(batch, num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sm_scale);
  if (st != PKC_OK) return st;
  if ((st = check_prefix_supported(dtype, page_size)) != PKC_OK) return st;
  if (fp8 && (st = check_fp8(dtype, k_scale, v_scale)) != PKC_OK) return st;
  if (!dtype_ok(o_dtype)) return fail(PKC_ERR_UNSUPPORTED, "unknown o_dtype");
  if (!plan || !level_dev) return fail(PKC_ERR_INVALID_ARG, "plan and level_dev are required");
  if ((st = check_plan(plan, batch, num_qo_heads, num_kv_heads, head_dim, page_size, dev_ws, dev_bytes)) != PKC_OK)
    return st;
  if (level < 0 || level >= plan->num_levels) return fail(PKC_ERR_INVALID_ARG, "level out of range");
  if (batch == 0) return PKC_OK;
  if (!q || !k_pool || !v_pool || !o_state || !lse_state) return fail(PKC_ERR_INVALID_ARG, "NULL tensor pointer");
  if (num_pages < 1) return fail(PKC_ERR_INVALID_ARG, "num_pages must be >= 1 (masked lanes read row 0 of page 0)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = run_level(plan, level, q, k_pool, v_pool, num_pages, level_dev, dtype, sm_scale, dev_ws, s,
                      fp8, k_scale, v_scale, nullptr, plan->host_src != 0)) != PKC_OK)
    return st;
  pkc::MergePlanParams m = merge_params(plan, dev_ws, level, level + 1, false, o_state, lse_state);
  return timed(2, s, "merge kernel launch", [&] { return pkc::launch_merge_plan(o_dtype, head_dim, m, s); });
}

pkc_status pkc_prefix_attention(const pkc_plan_info* plan, int32_t level, const void* q,
                                const void* k_pool, const void* v_pool, int64_t num_pages,
                                const pkc_level_dev* level_dev, int32_t batch,
                                int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t page_size, pkc_dtype dtype, float sm_scale,
                                void* o_state, pkc_dtype o_dtype, float* lse_state,
                                void* dev_ws, size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return prefix_impl(false, 1.f, 1.f, plan, level, q, k_pool, v_pool, num_pages, level_dev, batch,
                     num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sm_scale, o_state,
                     o_dtype, lse_state, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_prefix_attention")
}

pkc_status pkc_prefix_attention_fp8(const pkc_plan_info* plan, int32_t level, const void* q,
                                    const void* k_pool, const void* v_pool, float k_scale,
                                    float v_scale, int64_t num_pages,
                                    const pkc_level_dev* level_dev, int32_t batch,
                                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_size, pkc_dtype q_dtype, float sm_scale,
                                    void* o_state, pkc_dtype o_dtype, float* lse_state,
                                    void* dev_ws, size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return prefix_impl(true, k_scale, v_scale, plan, level, q, k_pool, v_pool, num_pages, level_dev,
                     batch, num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, sm_scale,
                     o_state, o_dtype, lse_state, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_prefix_attention_fp8")
}

static pkc_status prefill_impl(bool fp8, float k_scale, float v_scale, const pkc_plan_info* plan,
                               const void* q, const void* k_pool, const void* v_pool,
                               int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                               const int32_t* qo_indptr, const int32_t* kv_lens,
                               int32_t num_requests, int32_t total_q, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               pkc_dtype dtype, float sm_scale, int32_t causal, void* o,
                               float* lse, void* dev_ws, size_t dev_bytes, void* stream,
                               const uint8_t* tree_mask = nullptr, const int32_t* mask_indptr = nullptr,
                               int32_t mask_bytes = 0) {
  pkc_status st = check_shapes(total_q, num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sm_scale);
  if (st != PKC_OK) return st;
  if ((st = check_prefix_supported(dtype, page_size)) != PKC_OK) return st;
  if (fp8 && (st = check_fp8(dtype, k_scale, v_scale)) != PKC_OK) return st;
  if (!plan) return fail(PKC_ERR_INVALID_ARG, "batch prefill needs a plan");
  if (num_requests < 0) return fail(PKC_ERR_INVALID_ARG, "num_requests < 0");
  if ((st = check_plan(plan, total_q, num_qo_heads, num_kv_heads, head_dim, page_size, dev_ws, dev_bytes)) != PKC_OK)
    return st;
  if (plan->num_levels != 1 || plan->lvl_groups[0] != num_requests || plan->dec_items != 0)
    return fail(PKC_ERR_PLAN_MISMATCH,
                "batch prefill needs a plan with batch = total_q, one level whose groups are the "
                "requests and no decode items");
  if (plan->lvl_causal[0] != (causal ? 1 : 0))
    return fail(PKC_ERR_PLAN_MISMATCH,
                "the plan's level was built with a different causal flag (a causal plan covers "
                "only the tokens each tile's queries see)");
  if (total_q == 0) return PKC_OK;
  if (!q || !k_pool || !v_pool || !o || !lse || !block_table || !qo_indptr || !kv_lens)
    return fail(PKC_ERR_INVALID_ARG, "NULL pointer");
  if (num_pages < 1 || max_blocks < 1)
    return fail(PKC_ERR_INVALID_ARG, "num_pages and max_blocks must be >= 1");
  if ((int64_t)max_blocks * page_size > INT32_MAX || (int64_t)max_blocks * num_requests > INT32_MAX)
    return fail(PKC_ERR_INVALID_ARG, "block table too large for int32 offsets");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (tree_mask && (!causal || !mask_indptr || mask_bytes < 0))
    return fail(PKC_ERR_INVALID_ARG, "tree masks refine the causal mask: they need causal = 1, "
                                     "mask_indptr and mask_bytes >= 0");
  const PrefillLevel pf{block_table, max_blocks, qo_indptr, kv_lens, causal ? 1 : 0, o, lse,
                        tree_mask, mask_indptr, mask_bytes};
  if ((st = run_level(plan, 0, q, k_pool, v_pool, num_pages, nullptr, dtype, sm_scale, dev_ws, s, fp8,
                      k_scale, v_scale, &pf, plan->host_src != 0)) != PKC_OK)
    return st;
  // Query rows written through by their tile's only item are flagged and skipped; the merge is
  // enqueued even when every row is (launches independent of the plan's lengths).
  pkc::MergePlanParams m = merge_params(plan, dev_ws, 0, 1, true, o, lse);
  return timed(2, s, "merge kernel launch", [&] { return pkc::launch_merge_plan(dtype, head_dim, m, s); });
}

pkc_status pkc_batch_prefill_paged(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                   const void* v_pool, int64_t num_pages,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* qo_indptr, const int32_t* kv_lens,
                                   int32_t num_requests, int32_t total_q, int32_t num_qo_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                   pkc_dtype dtype, float sm_scale, int32_t causal, void* o,
                                   float* lse, void* dev_ws, size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return prefill_impl(false, 1.f, 1.f, plan, q, k_pool, v_pool, num_pages, block_table, max_blocks,
                      qo_indptr, kv_lens, num_requests, total_q, num_qo_heads, num_kv_heads, head_dim,
                      page_size, dtype, sm_scale, causal, o, lse, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_batch_prefill_paged")
}

pkc_status pkc_batch_prefill_paged_tree(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_pages,
                                        const int32_t* block_table, int32_t max_blocks,
                                        const int32_t* qo_indptr, const int32_t* kv_lens,
                                        const uint8_t* tree_mask, const int32_t* mask_indptr,
                                        int32_t mask_bytes, int32_t num_requests, int32_t total_q,
                                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t page_size, pkc_dtype dtype, float sm_scale, void* o,
                                        float* lse, void* dev_ws, size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  if (!tree_mask) return fail(PKC_ERR_INVALID_ARG, "tree_mask is NULL");
  return prefill_impl(false, 1.f, 1.f, plan, q, k_pool, v_pool, num_pages, block_table, max_blocks,
                      qo_indptr, kv_lens, num_requests, total_q, num_qo_heads, num_kv_heads, head_dim,
                      page_size, dtype, sm_scale, 1, o, lse, dev_ws, dev_bytes, stream, tree_mask,
                      mask_indptr, mask_bytes);
  PKC_TRY_END("pkc_batch_prefill_paged_tree")
}

pkc_status pkc_batch_prefill_paged_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                       const void* v_pool, float k_scale, float v_scale,
                                       int64_t num_pages, const int32_t* block_table,
                                       int32_t max_blocks, const int32_t* qo_indptr,
                                       const int32_t* kv_lens, int32_t num_requests,
                                       int32_t total_q, int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                       float sm_scale, int32_t causal, void* o, float* lse,
                                       void* dev_ws, size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return prefill_impl(true, k_scale, v_scale, plan, q, k_pool, v_pool, num_pages, block_table,
                      max_blocks, qo_indptr, kv_lens, num_requests, total_q, num_qo_heads, num_kv_heads,
                      head_dim, page_size, q_dtype, sm_scale, causal, o, lse, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_batch_prefill_paged_fp8")
}

pkc_status pkc_merge_states(const void* o_states, pkc_dtype in_dtype, const float* lse_states,
                            int32_t num_states, const int32_t* indptr, const int32_t* indices,
                            int32_t num_outputs, int32_t states_per_output, int32_t num_heads,
                            int32_t head_dim, void* o_out, pkc_dtype out_dtype, float* lse_out,
                            void* stream) {
  PKC_TRY_BEGIN
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(PKC_ERR_UNSUPPORTED, "unknown dtype");
  if (!(head_dim == 64 || head_dim == 128)) return fail(PKC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_states < 0 || num_outputs < 0 || num_heads <= 0)
    return fail(PKC_ERR_INVALID_ARG, "bad num_states / num_outputs / num_heads");
  if (num_outputs == 0) return PKC_OK;
  if (!o_out || !lse_out) return fail(PKC_ERR_INVALID_ARG, "NULL output pointer");
  if (num_states > 0 && (!o_states || !lse_states)) return fail(PKC_ERR_INVALID_ARG, "NULL state pointer");
  if (!indptr) {
    if (indices) return fail(PKC_ERR_INVALID_ARG, "indices without indptr");
    if (states_per_output < 0 || (int64_t)states_per_output * num_outputs > num_states)
      return fail(PKC_ERR_INVALID_ARG, "states_per_output * num_outputs exceeds num_states");
  }
  pkc::MergeGenericParams p{};
  p.o_states = o_states;
  p.lse_states = lse_states;
  p.num_states = num_states;
  p.indptr = indptr;
  p.indices = indices;
  p.num_outputs = num_outputs;
  p.states_per_output = states_per_output;
  p.num_heads = num_heads;
  p.o_out = o_out;
  p.lse_out = lse_out;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return timed(3, s, "merge kernel launch", [&] { return pkc::launch_merge_generic(in_dtype, out_dtype, head_dim, p, s); });
  PKC_TRY_END("pkc_merge_states")
}

pkc_status pkc_merge_state_inplace(void* o_a, float* lse_a, const void* o_b, const float* lse_b,
                                   int32_t num_rows, int32_t num_heads, int32_t head_dim,
                                   pkc_dtype dtype, void* stream) {
  PKC_TRY_BEGIN
  if (!dtype_ok(dtype)) return fail(PKC_ERR_UNSUPPORTED, "unknown dtype");
  if (!(head_dim == 64 || head_dim == 128)) return fail(PKC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_rows < 0 || num_heads <= 0) return fail(PKC_ERR_INVALID_ARG, "bad num_rows / num_heads");
  if (num_rows == 0) return PKC_OK;
  if (!o_a || !lse_a || !o_b || !lse_b) return fail(PKC_ERR_INVALID_ARG, "NULL pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return timed(3, s, "merge kernel launch", [&] {
    return pkc::launch_merge_inplace(dtype, head_dim, o_a, lse_a, o_b, lse_b, (int64_t)num_rows * num_heads, s);
  });
  PKC_TRY_END("pkc_merge_state_inplace")
}

static pkc_status cascade_impl(bool fp8, float k_scale, float v_scale, const pkc_plan_info* plan,
                               const void* q, const void* k_pool, const void* v_pool,
                               int64_t num_pages, const pkc_level_dev* levels, int32_t num_levels,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* suffix_seqlens, int32_t batch, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               pkc_dtype dtype, float sm_scale, void* o, float* lse, void* dev_ws,
                               size_t dev_bytes, void* stream) {
  pkc_status st = check_shapes(batch, num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sm_scale);
  if (st != PKC_OK) return st;
  if (fp8 && (st = check_fp8(dtype, k_scale, v_scale)) != PKC_OK) return st;
  if (!plan) return fail(PKC_ERR_INVALID_ARG, "cascade decode needs a plan");
  if ((st = check_plan(plan, batch, num_qo_heads, num_kv_heads, head_dim, page_size, dev_ws, dev_bytes)) != PKC_OK)
    return st;
  if (num_levels != plan->num_levels) return fail(PKC_ERR_PLAN_MISMATCH, "num_levels differs from the plan");
  if (num_levels > 0) {
    if (!levels) return fail(PKC_ERR_INVALID_ARG, "levels is NULL");
    if ((st = check_prefix_supported(dtype, page_size)) != PKC_OK) return st;
  }
  if (batch == 0) return PKC_OK;
  if (!q || !k_pool || !v_pool || !o || !lse) return fail(PKC_ERR_INVALID_ARG, "NULL tensor pointer");
  if (plan->dec_items > 0 && !block_table) return fail(PKC_ERR_INVALID_ARG, "block_table is NULL");
  if (num_pages < 1 || max_blocks < 0)
    return fail(PKC_ERR_INVALID_ARG, "num_pages must be >= 1 (masked lanes read row 0 of page 0) and max_blocks >= 0");
  if ((int64_t)max_blocks * page_size > INT32_MAX)
    return fail(PKC_ERR_INVALID_ARG, "max_blocks * page_size exceeds int32");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // A deferred plan comes over with the first level kernel (or ahead of the decode kernel when
  // the cascade has no level).
  if (num_levels == 0 && (st = upload_if_deferred(plan, dev_ws, s)) != PKC_OK) return st;
  for (int32_t l = 0; l < num_levels; ++l)
    if ((st = run_level(plan, l, q, k_pool, v_pool, num_pages, &levels[l], dtype, sm_scale, dev_ws, s,
                        fp8, k_scale, v_scale, nullptr, l == 0 && plan->host_src != 0)) != PKC_OK)
      return st;
  pkc::DecodeParams p = decode_params(q, k_pool, v_pool, num_pages, block_table, max_blocks,
                                      suffix_seqlens, nullptr, num_qo_heads, num_kv_heads,
                                      page_size, sm_scale, o, lse);
  if (fp8) {
    p.scale_log2 *= k_scale;
    p.v_scale = v_scale;
  }
  p.st_o = at<float>(dev_ws, plan->off_state_o);
  p.st_lse = at<float>(dev_ws, plan->off_state_lse);
  p.indptr = at<int32_t>(dev_ws, plan->off_dec_indptr);
  p.items = at<int32_t>(dev_ws, plan->off_dec_items);
  if (num_levels > 0) {
    // Items that finish their request fold in the request's level states.
    p.merge_ptr = at<int32_t>(dev_ws, plan->off_merge_ptr);
    p.merge_rows = at<int32_t>(dev_ws, plan->off_merge_rows);
    p.nl2 = num_levels + 2;
    p.num_levels = num_levels;
    for (int32_t l = 0; l < num_levels; ++l) p.lvl_tile_q[l] = plan->lvl_tile_q[l];
    p.req_levels = at<int32_t>(dev_ws, plan->off_req_levels);
    // Bounds of the state buffers for the fold's buffer loads: the workspace's capacity (fixed
    // by the parameters and level shapes, like every other launch argument).
    const int64_t o_bytes = plan->off_state_lse - plan->off_state_o;
    const int64_t lse_bytes = plan->dev_bytes - plan->off_state_lse;
    if (o_bytes <= INT32_MAX && lse_bytes <= INT32_MAX) {
      p.fold_o_bytes = (int32_t)o_bytes;
      p.fold_lse_bytes = (int32_t)lse_bytes;
    }
  }
  if (plan->dec_contraction == 1) set_contraction(&p, plan, dev_ws, num_levels);
  const int g = num_qo_heads / num_kv_heads;
  if ((st = timed(0, s, "decode kernel launch", [&] {
         return fp8 ? pkc::launch_decode_fp8(dtype, head_dim, g, plan->dec_waves, p, plan->num_ctas, s)
                    : pkc::launch_decode(dtype, head_dim, g, plan->dec_waves, p, plan->num_ctas, s);
       })) != PKC_OK)
    return st;
  if (plan->dec_contraction == 1) return PKC_OK;   // the decode kernel merged every request
  // Always enqueued (it skips the requests finished by the decode kernel): the launches of a run
  // do not depend on the plan's lengths, so a captured run stays valid across re-plans.
  pkc::MergePlanParams m = merge_params(plan, dev_ws, 0, num_levels + 1, true, o, lse);
  return timed(2, s, "merge kernel launch", [&] { return pkc::launch_merge_plan(dtype, head_dim, m, s); });
}

pkc_status pkc_cascade_decode(const pkc_plan_info* plan, const void* q, const void* k_pool,
                              const void* v_pool, int64_t num_pages,
                              const pkc_level_dev* levels, int32_t num_levels,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* suffix_seqlens, int32_t batch, int32_t num_qo_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              pkc_dtype dtype, float sm_scale, void* o, float* lse, void* dev_ws,
                              size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return cascade_impl(false, 1.f, 1.f, plan, q, k_pool, v_pool, num_pages, levels, num_levels,
                      block_table, max_blocks, suffix_seqlens, batch, num_qo_heads, num_kv_heads,
                      head_dim, page_size, dtype, sm_scale, o, lse, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_cascade_decode")
}

pkc_status pkc_cascade_decode_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                  const void* v_pool, float k_scale, float v_scale,
                                  int64_t num_pages, const pkc_level_dev* levels,
                                  int32_t num_levels, const int32_t* block_table,
                                  int32_t max_blocks, const int32_t* suffix_seqlens,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                  float sm_scale, void* o, float* lse, void* dev_ws,
                                  size_t dev_bytes, void* stream) {
  PKC_TRY_BEGIN
  return cascade_impl(true, k_scale, v_scale, plan, q, k_pool, v_pool, num_pages, levels, num_levels,
                      block_table, max_blocks, suffix_seqlens, batch, num_qo_heads, num_kv_heads,
                      head_dim, page_size, q_dtype, sm_scale, o, lse, dev_ws, dev_bytes, stream);
  PKC_TRY_END("pkc_cascade_decode_fp8")
}

pkc_status pkc_debug_gather_rows(const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* cache_seqlens, const int32_t* kv_start,
                                 int32_t batch, int32_t page_size, int64_t num_pages,
                                 int32_t* rows_out, int32_t max_tokens, void* stream) {
  PKC_TRY_BEGIN
  if (batch < 0 || max_blocks < 0 || max_tokens < 0 || num_pages < 0)
    return fail(PKC_ERR_INVALID_ARG, "bad sizes");
  if (!pkc::is_pow2(page_size) || page_size > 1024) return fail(PKC_ERR_UNSUPPORTED, "bad page_size");
  if ((int64_t)max_blocks * page_size > INT32_MAX) return fail(PKC_ERR_INVALID_ARG, "table too large");
  if (batch == 0 || max_tokens == 0) return PKC_OK;
  if (!block_table || !cache_seqlens || !rows_out) return fail(PKC_ERR_INVALID_ARG, "NULL pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = pkc::launch_debug_gather(block_table, max_blocks, cache_seqlens, kv_start, batch,
                                          log2i(page_size), num_pages, rows_out, max_tokens, s);
  if (e != hipSuccess) return hip_fail(e, "debug gather launch");
  return PKC_OK;
  PKC_TRY_END("pkc_debug_gather_rows")
}

pkc_status pkc_debug_cta_trace(const pkc_plan_info* plan, int32_t stage, const void* dev_ws,
                               int32_t* trace_out, int64_t trace_len,
                               int32_t max_items_per_cta, void* stream) {
  PKC_TRY_BEGIN
  if (!plan || plan->magic != PKC_PLAN_MAGIC) return fail(PKC_ERR_INVALID_ARG, "bad plan");
  if (!dev_ws || plan->dev_ws != (uint64_t)(uintptr_t)dev_ws)
    return fail(PKC_ERR_PLAN_MISMATCH, "plan was copied to another device workspace");
  if (stage < 0 || stage > plan->num_levels) return fail(PKC_ERR_INVALID_ARG, "stage out of range");
  if (max_items_per_cta <= 0 || !trace_out) return fail(PKC_ERR_INVALID_ARG, "bad trace buffer");
  const bool dec = stage == plan->num_levels;
  const int32_t ctas = dec ? plan->num_ctas : plan->level_ctas;
  if (trace_len < (int64_t)ctas * max_items_per_cta * 8)
    return fail(PKC_ERR_WORKSPACE_TOO_SMALL, "trace buffer too small");
  void* ws = const_cast<void*>(dev_ws);
  pkc_status st = upload_if_deferred(plan, ws, reinterpret_cast<hipStream_t>(stream));
  if (st != PKC_OK) return st;
  const int32_t* indptr = at<int32_t>(ws, dec ? plan->off_dec_indptr : plan->off_lvl_indptr[stage]);
  const int32_t* items = at<int32_t>(ws, dec ? plan->off_dec_items : plan->off_lvl_items[stage]);
  hipError_t e = pkc::launch_debug_trace(indptr, items, ctas, trace_out, max_items_per_cta,
                                         reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "debug trace launch");
  return PKC_OK;
  PKC_TRY_END("pkc_debug_cta_trace")
}

pkc_status pkc_append_kv(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* cache_seqlens, int32_t* new_seqlens, int32_t batch,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                         pkc_dtype dtype, void* stream) {
  PKC_TRY_BEGIN
  if (batch < 0 || num_kv_heads <= 0 || max_blocks < 0 || num_pages < 0)
    return fail(PKC_ERR_INVALID_ARG, "append: bad sizes");
  if (!(head_dim == 64 || head_dim == 128)) return fail(PKC_ERR_UNSUPPORTED, "append: head_dim must be 64 or 128");
  if (!pkc::is_pow2(page_size) || page_size > 1024)
    return fail(PKC_ERR_UNSUPPORTED, "append: page_size must be a power of two in [1, 1024]");
  if (dtype != PKC_F32 && dtype != PKC_F16 && dtype != PKC_BF16) return fail(PKC_ERR_UNSUPPORTED, "append: dtype");
  if (batch == 0) return PKC_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !cache_seqlens)
    return fail(PKC_ERR_INVALID_ARG, "append: NULL pointer");
  pkc::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.num_pages = num_pages;
  p.block_table = block_table;
  p.max_blocks = max_blocks;
  p.page_shift = log2i(page_size);
  p.seqlens = cache_seqlens;
  p.seqlens_out = new_seqlens;
  p.row_bytes = (int64_t)num_kv_heads * head_dim * (dtype == PKC_F32 ? 4 : 2);
  hipError_t e = pkc::launch_append_kv(p, batch, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PKC_OK;
  PKC_TRY_END("pkc_append_kv")
}

pkc_status pkc_append_kv_ragged(const void* k_new, const void* v_new, int64_t total_new,
                                const int32_t* new_indptr, void* k_pool, void* v_pool,
                                int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* cache_seqlens, int32_t* new_seqlens, int32_t batch,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                pkc_dtype dtype, void* stream) {
  PKC_TRY_BEGIN
  if (batch < 0 || batch > 65535 || num_kv_heads <= 0 || max_blocks < 0 || num_pages < 0 || total_new < 0)
    return fail(PKC_ERR_INVALID_ARG, "append: bad sizes (batch must be in [0, 65535])");
  if (!(head_dim == 64 || head_dim == 128)) return fail(PKC_ERR_UNSUPPORTED, "append: head_dim must be 64 or 128");
  if (!pkc::is_pow2(page_size) || page_size > 1024)
    return fail(PKC_ERR_UNSUPPORTED, "append: page_size must be a power of two in [1, 1024]");
  if (dtype != PKC_F32 && dtype != PKC_F16 && dtype != PKC_BF16) return fail(PKC_ERR_UNSUPPORTED, "append: dtype");
  if (batch == 0) return PKC_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !cache_seqlens || !new_indptr)
    return fail(PKC_ERR_INVALID_ARG, "append: NULL pointer");
  if (new_seqlens == cache_seqlens)
    return fail(PKC_ERR_INVALID_ARG, "append: new_seqlens must not alias cache_seqlens (several "
                                     "workgroups of a request read its old length)");
  pkc::AppendRaggedParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.num_pages = num_pages;
  p.block_table = block_table;
  p.max_blocks = max_blocks;
  p.page_shift = log2i(page_size);
  p.seqlens = cache_seqlens;
  p.new_indptr = new_indptr;
  p.total_new = total_new;
  p.seqlens_out = new_seqlens;
  p.row_bytes = (int64_t)num_kv_heads * head_dim * (dtype == PKC_F32 ? 4 : 2);
  hipError_t e = pkc::launch_append_kv_ragged(p, batch, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PKC_OK;
  PKC_TRY_END("pkc_append_kv_ragged")
}

pkc_status pkc_read_stream_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_len,
                                 void* stream) {
  PKC_TRY_BEGIN
  constexpr int64_t kMiB = 1 << 20;
  if (!src || !sink || bytes <= 0 || bytes % kMiB)
    return fail(PKC_ERR_INVALID_ARG, "read probe: src and sink must be set, bytes a positive multiple of 1 MiB");
  if (reinterpret_cast<uintptr_t>(src) & 15) return fail(PKC_ERR_INVALID_ARG, "read probe: src must be 16-byte aligned");
  if (sink_len < bytes / kMiB * 256) return fail(PKC_ERR_WORKSPACE_TOO_SMALL, "read probe: sink too small");
  hipError_t e = pkc::launch_read_stream(src, bytes / kMiB, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  return PKC_OK;
  PKC_TRY_END("pkc_read_stream_probe")
}

pkc_status pkc_timing_enable(int32_t enable) {
  g_timing = enable != 0;
  return PKC_OK;
}

pkc_status pkc_timing_reset(void) {
  PKC_TRY_BEGIN
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& t : g_pending) {
    (void)hipEventSynchronize(t.stop);
    g_free_events.push_back(t.start);
    g_free_events.push_back(t.stop);
  }
  g_pending.clear();
  for (int i = 0; i < 4; ++i) {
    g_launches[i] = 0;
    g_ms[i] = 0;
  }
  return PKC_OK;
  PKC_TRY_END("pkc_timing_reset")
}

pkc_status pkc_timing_read(int32_t kind, int64_t* launches, double* total_ms) {
  PKC_TRY_BEGIN
  if (kind < 0 || kind > 3) return fail(PKC_ERR_INVALID_ARG, "kind must be 0..3");
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& t : g_pending) {
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, t.start, t.stop)) != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    g_launches[t.kind] += 1;
    g_ms[t.kind] += ms;
    g_free_events.push_back(t.start);
    g_free_events.push_back(t.stop);
  }
  g_pending.clear();
  if (launches) *launches = g_launches[kind];
  if (total_ms) *total_ms = g_ms[kind];
  return PKC_OK;
  PKC_TRY_END("pkc_timing_read")
}

}  // extern "C"
