// Host-only load-balancing plan: declarations shared by plan.cpp and api.cpp.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pkc.h"

namespace pkc {

// Thread-local error message helpers (defined in plan.cpp).
pkc_status fail(pkc_status s, const std::string& msg);
void clear_error();

// One work item of a stage, 8 int32 as stored in the workspace.
struct Item {
  int32_t req;    // request (decode stage) or group (cascade level)
  int32_t q0;     // first query (request index) of the tile
  int32_t nq;     // queries in the tile
  int32_t kb;     // KV chunk [kb, ke) inside the tile's KV, tokens
  int32_t ke;
  int32_t row;    // first state row, or -1 = write-through
  int32_t tile;   // query tile index inside the request / group
  int32_t w;      // work index (enumeration order)
};
static_assert(sizeof(Item) == 32, "item record is 8 int32");

// A stage's plan.  Stage objects are reused from one plan to the next (a serving loop plans
// every step), so their vectors keep their capacity: only cta[0 .. ctas) is meaningful.
struct Stage {
  int32_t ctas = 0;
  int32_t tile_q = 1;
  int32_t kv_chunk = 1;
  std::vector<Item> items;                  // by w
  std::vector<std::vector<int32_t>> cta;    // per CTA: w in assignment order
  std::vector<int64_t> cta_cost;
  std::vector<int32_t> order;               // scratch: items sorted longest first
  std::vector<std::pair<int64_t, int32_t>> heap;   // scratch: the (cost, CTA) queue
};

// Steps 1-7 of the scheduler for one stage. qo_lens may be nullptr (all 1).  causal: a query
// tile's KV is only the part its last query sees under the causal mask.
pkc_status lpt_plan(const int32_t* qo_lens, const int32_t* kv_lens, int32_t n, int32_t tile_q,
                    int32_t ctas, int64_t alpha, int64_t beta, int32_t chunk_align,
                    bool enable_split, Stage* out, bool causal = false);

// Offsets of every array of a plan inside the host buffer / device workspace; fixed by the
// parameters and the level shapes only, so they do not move from one step to the next.
struct Layout {
  int64_t off_dec_indptr, off_dec_items, off_merge_ptr, off_merge_rows, off_req_flags, off_req_levels;
  int64_t off_counters;
  int64_t off_lvl_indptr[PKC_MAX_LEVELS], off_lvl_items[PKC_MAX_LEVELS];
  int64_t int_bytes;
  int64_t max_dec_items, max_lvl_items[PKC_MAX_LEVELS];
  int64_t max_merge_rows;
  int64_t max_state_rows;
  int64_t max_dec_rows, max_lvl_rows[PKC_MAX_LEVELS];
  int64_t off_state_o, off_state_lse, dev_bytes;
};

struct Resolved {
  pkc_plan_params p;
  int32_t group;  // Hq / Hkv
};

pkc_status check_params(const pkc_plan_params* params, bool need_ctas, Resolved* out);
pkc_status check_levels(const pkc_level_host* levels, int32_t num_levels, int32_t batch,
                        bool need_kv_lens);
pkc_status compute_layout(const Resolved& r, const pkc_level_host* levels, int32_t num_levels,
                          Layout* lay);

// Builds the whole plan into host_buf and fills *out (dev_ws = 0).
pkc_status build_plan_host(const Resolved& r, const int32_t* kv_lens_h,
                           const pkc_level_host* levels, int32_t num_levels, void* host_buf,
                           size_t host_bytes, pkc_plan_info* out);

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace pkc
