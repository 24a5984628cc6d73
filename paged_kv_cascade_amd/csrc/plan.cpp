// CPU load-balancing plan (host C++, no HIP calls).
//
// Implements the scheduler of "FlashInfer: Efficient and Customizable Attention Engine for
// LLM Inference Serving" (paper summary, section A3, "load-balancing scheduling") and the
// workspace rules of its appendix D:
//   * cost of a tile: alpha * l_q + beta * l_kv (integers here);
//   * maximum chunk L_kv = ceil(sum_i ceil(l_qo(i) / T_q) * l_kv(i) / #CTA), at least 1,
//     rounded up to chunk_align;
//   * each query tile's KV is cut greedily into chunks of at most L_kv, work index w in
//     (request, tile, chunk) order; the list is sorted longest first with a stable sort;
//   * a min-priority queue of (cost, CTA), ties to the smaller CTA index, receives the items
//     in that order;
//   * tiles with a single chunk write their state straight to the final output
//     (write-through); every other item gets the next partial-state slot in ascending w.
//     Cascade levels always write states (they are merged with the suffix), except when the
//     caller asks for level write-through (batch prefill): then a level tile with a single
//     chunk, in a plan with one level whose group has no own KV, writes the final output too;
//   * buffers are sized from upper bounds so that their addresses never change.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "plan_core.h"

namespace pkc {

static thread_local std::string g_last_error;

pkc_status fail(pkc_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
void clear_error() { g_last_error.clear(); }

}  // namespace pkc

extern "C" const char* pkc_last_error(void) { return pkc::g_last_error.c_str(); }

namespace pkc {

pkc_status lpt_plan(const int32_t* qo_lens, const int32_t* kv_lens, int32_t n, int32_t tile_q,
                    int32_t ctas, int64_t alpha, int64_t beta, int32_t chunk_align,
                    bool enable_split, Stage* out, bool causal) {
  if (tile_q < 1 || ctas < 1 || chunk_align < 1 || n < 0)
    return fail(PKC_ERR_INVALID_ARG, "plan: tile_q, ctas and chunk_align must be >= 1");
  if (alpha < 0 || beta < 0) return fail(PKC_ERR_INVALID_ARG, "plan: alpha, beta must be >= 0");
  if (n > 0 && kv_lens == nullptr) return fail(PKC_ERR_INVALID_ARG, "plan: kv_lens is NULL");
  auto lqo = [&](int32_t i) -> int64_t { return qo_lens ? qo_lens[i] : 1; };
  // KV extent of query tile j of request i: all of it, or with the causal mask the tokens
  // its last query sees (the request's queries are its last l_qo tokens).
  auto extent = [&](int32_t i, int64_t j) -> int64_t {
    if (!causal) return kv_lens[i];
    const int64_t last = std::min<int64_t>((j + 1) * tile_q, lqo(i));   // queries before the end
    return std::min<int64_t>(kv_lens[i], std::max<int64_t>(0, (int64_t)kv_lens[i] - lqo(i) + last));
  };
  int64_t total = 0, longest = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lqo(i) < 0 || kv_lens[i] < 0) return fail(PKC_ERR_INVALID_ARG, "plan: negative length");
    for (int64_t j = 0; j < ceil_div(lqo(i), tile_q); ++j) total += extent(i, j);
    longest = std::max<int64_t>(longest, kv_lens[i]);
  }
  // Step 3: maximum KV chunk length.
  int64_t L = enable_split ? std::max<int64_t>(1, ceil_div(total, ctas)) : std::max<int64_t>(1, longest);
  L = align_up(L, chunk_align);
  if (L > INT32_MAX) return fail(PKC_ERR_INVALID_ARG, "plan: chunk length overflows int32");

  Stage& st = *out;
  st.ctas = ctas;
  st.tile_q = tile_q;
  st.kv_chunk = (int32_t)L;
  st.items.clear();
  // Step 4: chunks of every query tile, w in (request, tile, chunk) order.
  for (int32_t i = 0; i < n; ++i) {
    const int64_t tiles = ceil_div(lqo(i), tile_q);
    for (int64_t j = 0; j < tiles; ++j) {
      const int32_t lq = (int32_t)std::min<int64_t>(tile_q, lqo(i) - j * tile_q);
      const int64_t ext = extent(i, j);
      const int64_t chunks = ceil_div(ext, L);
      for (int64_t c = 0; c < chunks; ++c) {
        Item it;
        it.req = i;
        it.q0 = (int32_t)(j * tile_q);  // relative to the request / group; fixed up by caller
        it.nq = lq;
        it.kb = (int32_t)(c * L);
        it.ke = (int32_t)std::min<int64_t>((c + 1) * L, ext);
        it.row = -1;
        it.tile = (int32_t)j;
        it.w = (int32_t)st.items.size();
        st.items.push_back(it);
      }
    }
  }
  // Step 5: longest first, stable (equal lengths keep ascending w).
  std::vector<int32_t>& order = st.order;
  order.resize(st.items.size());
  std::iota(order.begin(), order.end(), 0);
  bool sorted = true;
  for (size_t i = 1; i < order.size() && sorted; ++i)
    sorted = (st.items[i - 1].ke - st.items[i - 1].kb) >= (st.items[i].ke - st.items[i].kb);
  if (!sorted)
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return (st.items[a].ke - st.items[a].kb) > (st.items[b].ke - st.items[b].kb);
    });
  // Steps 6-7: min-cost CTA first, ties to the smaller index (a min-heap on (cost, CTA)).
  using Entry = std::pair<int64_t, int32_t>;
  std::vector<Entry>& heap = st.heap;
  heap.resize(ctas);
  for (int32_t c = 0; c < ctas; ++c) heap[c] = {0, c};   // already a valid min-heap
  if ((int32_t)st.cta.size() < ctas) st.cta.resize(ctas);
  for (int32_t c = 0; c < ctas; ++c) st.cta[c].clear();
  st.cta_cost.assign(ctas, 0);
  const auto later = std::greater<Entry>();
  for (int32_t w : order) {
    std::pop_heap(heap.begin(), heap.end(), later);
    Entry& e = heap.back();
    const Item& it = st.items[w];
    st.cta[e.second].push_back(w);
    e.first += alpha * it.nq + beta * (int64_t)(it.ke - it.kb);
    st.cta_cost[e.second] = e.first;
    std::push_heap(heap.begin(), heap.end(), later);
  }
  return PKC_OK;
}

pkc_status check_params(const pkc_plan_params* params, bool need_ctas, Resolved* out) {
  if (!params) return fail(PKC_ERR_INVALID_ARG, "params is NULL");
  const pkc_plan_params& p = *params;
  if (p.batch < 0) return fail(PKC_ERR_INVALID_ARG, "batch must be >= 0");
  if (p.num_qo_heads <= 0 || p.num_kv_heads <= 0 || p.num_qo_heads % p.num_kv_heads)
    return fail(PKC_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  const int32_t g = p.num_qo_heads / p.num_kv_heads;
  if (!(g == 1 || g == 2 || g == 4 || g == 8))
    return fail(PKC_ERR_UNSUPPORTED, "group size Hq/Hkv must be 1, 2, 4 or 8");
  if (!(p.head_dim == 64 || p.head_dim == 128))
    return fail(PKC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!is_pow2(p.page_size) || p.page_size > 1024)
    return fail(PKC_ERR_UNSUPPORTED, "page_size must be a power of two in [1, 1024]");
  if (p.alpha < 0 || p.beta < 0) return fail(PKC_ERR_INVALID_ARG, "alpha and beta must be >= 0");
  if (p.chunk_align < 0) return fail(PKC_ERR_INVALID_ARG, "chunk_align must be >= 0");
  if (!(p.decode_waves == 0 || p.decode_waves == 1 || p.decode_waves == 2 || p.decode_waves == 4))
    return fail(PKC_ERR_INVALID_ARG, "decode_waves must be 0, 1, 2 or 4");
  if (!(p.level_write_through == 0 || p.level_write_through == 1))
    return fail(PKC_ERR_INVALID_ARG, "level_write_through must be 0 or 1");
  if (!(p.level_streams == 0 || p.level_streams == 1 || p.level_streams == 2))
    return fail(PKC_ERR_INVALID_ARG, "level_streams must be 0, 1 or 2");
  if (!(p.contraction == 0 || p.contraction == 1 || p.contraction == 2))
    return fail(PKC_ERR_INVALID_ARG, "contraction must be 0, 1 or 2");
  if (!(p.defer_upload == 0 || p.defer_upload == 1))
    return fail(PKC_ERR_INVALID_ARG, "defer_upload must be 0 or 1");
  if (p.num_ctas < 0 || p.level_ctas < 0 || p.level_tile_q < 0)
    return fail(PKC_ERR_INVALID_ARG, "num_ctas, level_ctas, level_tile_q must be >= 0");
  if (need_ctas && (p.num_ctas == 0 || p.level_ctas == 0))
    return fail(PKC_ERR_INVALID_ARG, "host-only plan needs explicit num_ctas and level_ctas");
  Resolved r;
  r.p = p;
  r.group = g;
  if (r.p.chunk_align == 0) r.p.chunk_align = 1;
  if (r.p.level_tile_q == 0) r.p.level_tile_q = 128 / g;
  if (r.p.level_tile_q * g > 128)
    return fail(PKC_ERR_UNSUPPORTED, "level_tile_q * (Hq/Hkv) must be <= 128 (rows of a prefix tile)");
  *out = r;
  return PKC_OK;
}

pkc_status check_levels(const pkc_level_host* levels, int32_t num_levels, int32_t batch,
                        bool need_kv_lens) {
  if (num_levels < 0 || num_levels > PKC_MAX_LEVELS)
    return fail(PKC_ERR_INVALID_ARG, "num_levels must be in [0, 8]");
  if (num_levels > 0 && !levels) return fail(PKC_ERR_INVALID_ARG, "levels is NULL");
  for (int32_t l = 0; l < num_levels; ++l) {
    const pkc_level_host& lv = levels[l];
    if (lv.num_groups < 0 || (lv.num_groups > 0 && !lv.qo_indptr))
      return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(l) + ": bad num_groups / qo_indptr");
    if (lv.num_groups == 0) continue;
    if (need_kv_lens && !lv.kv_lens)
      return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(l) + ": kv_lens is NULL");
    if (lv.qo_indptr[0] < 0) return fail(PKC_ERR_INVALID_ARG, "level qo_indptr[0] < 0");
    for (int32_t g = 0; g < lv.num_groups; ++g) {
      if (lv.qo_indptr[g + 1] < lv.qo_indptr[g])
        return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(l) + ": qo_indptr decreases");
      if (need_kv_lens && lv.kv_lens[g] < 0)
        return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(l) + ": negative kv_len");
    }
    if (lv.qo_indptr[lv.num_groups] > batch)
      return fail(PKC_ERR_INVALID_ARG, "level " + std::to_string(l) + ": qo_indptr[G] > batch");
  }
  return PKC_OK;
}

pkc_status compute_layout(const Resolved& r, const pkc_level_host* levels, int32_t num_levels,
                          Layout* lay) {
  const pkc_plan_params& p = r.p;
  const int64_t B = p.batch, NL = num_levels;
  int64_t off = 0;
  auto take = [&](int64_t ints) {
    int64_t o = off;
    off = align_up(off + ints * 4, 256);
    return o;
  };
  Layout L{};
  L.max_dec_items = (int64_t)p.num_ctas + B;
  L.max_dec_rows = NL > 0 ? L.max_dec_items : std::min<int64_t>(L.max_dec_items, 2 * (int64_t)p.num_ctas);
  L.off_dec_indptr = take(p.num_ctas + 1);
  L.off_dec_items = take(8 * L.max_dec_items);
  int64_t rows = 0, merge_rows = L.max_dec_rows;
  for (int32_t l = 0; l < num_levels; ++l) {
    int64_t tiles = 0;
    for (int32_t g = 0; g < levels[l].num_groups; ++g)
      tiles += ceil_div(levels[l].qo_indptr[g + 1] - levels[l].qo_indptr[g], p.level_tile_q);
    L.max_lvl_items[l] = (int64_t)p.level_ctas + tiles;
    L.max_lvl_rows[l] = L.max_lvl_items[l] * p.level_tile_q;
    rows += L.max_lvl_rows[l];
    merge_rows += L.max_lvl_rows[l];
    L.off_lvl_indptr[l] = take(p.level_ctas + 1);
    L.off_lvl_items[l] = take(8 * L.max_lvl_items[l]);
  }
  L.off_merge_ptr = take(B * (NL + 2));
  L.max_merge_rows = merge_rows;
  L.off_merge_rows = take(merge_rows);
  L.off_req_flags = take(B);
  L.off_req_levels = take(B * NL * 2 + 8);   // + padding: the decode kernel reads 4 levels' entries
  L.off_counters = take(B * (int64_t)p.num_kv_heads);   // zero in every plan
  L.int_bytes = off;
  L.max_state_rows = rows + L.max_dec_rows;
  const int64_t hd = (int64_t)p.num_qo_heads * p.head_dim;
  L.off_state_o = align_up(off, 256);
  L.off_state_lse = align_up(L.off_state_o + L.max_state_rows * hd * 4, 256);
  L.dev_bytes = align_up(L.off_state_lse + L.max_state_rows * p.num_qo_heads * 4, 256);
  if (L.max_state_rows > INT32_MAX || L.max_merge_rows > INT32_MAX)
    return fail(PKC_ERR_INVALID_ARG, "plan too large");
  *lay = L;
  return PKC_OK;
}

namespace {
// Working storage of build_plan_host, kept per thread so that a plan built every step reuses
// its vectors' capacity instead of allocating them again.
struct PlanScratch {
  std::vector<Stage> lv;
  Stage dec;
  std::vector<int32_t> flags, qo, chunks_of, chunks;
  std::vector<char> wt_group;
  std::vector<std::vector<int32_t>> per_req_lvl;
};
PlanScratch& plan_scratch() {
  static thread_local PlanScratch s;
  return s;
}
}  // namespace

pkc_status build_plan_host(const Resolved& r, const int32_t* kv_lens_h,
                           const pkc_level_host* levels, int32_t num_levels, void* host_buf,
                           size_t host_bytes, pkc_plan_info* out) {
  const pkc_plan_params& p = r.p;
  const int32_t B = p.batch;
  if (B > 0 && !kv_lens_h) return fail(PKC_ERR_INVALID_ARG, "kv_lens_h is NULL");
  if (!out) return fail(PKC_ERR_INVALID_ARG, "out is NULL");
  pkc_status s = check_levels(levels, num_levels, B, true);
  if (s != PKC_OK) return s;
  Layout L;
  if ((s = compute_layout(r, levels, num_levels, &L)) != PKC_OK) return s;
  if (!host_buf || host_bytes < (size_t)L.int_bytes)
    return fail(PKC_ERR_WORKSPACE_TOO_SMALL, "host buffer smaller than " + std::to_string(L.int_bytes) + " bytes");
  if (((uintptr_t)host_buf) & 15) return fail(PKC_ERR_INVALID_ARG, "host buffer must be 16-byte aligned");
  for (int32_t b = 0; b < B; ++b)
    if (kv_lens_h[b] < 0) return fail(PKC_ERR_INVALID_ARG, "negative kv_len for request " + std::to_string(b));

  char* base = static_cast<char*>(host_buf);
  std::memset(base, 0, (size_t)L.int_bytes);
  pkc_plan_info P{};
  P.magic = PKC_PLAN_MAGIC;
  P.batch = B;
  P.num_qo_heads = p.num_qo_heads;
  P.num_kv_heads = p.num_kv_heads;
  P.head_dim = p.head_dim;
  P.page_size = p.page_size;
  P.num_levels = num_levels;
  P.num_ctas = p.num_ctas;
  P.level_ctas = p.level_ctas;
  P.lvl_streams = p.level_streams;   // resolved from the device by pkc_plan (0 in host-only plans)
  // Automatic choice: with at most one decode CTA per request few requests are split, and
  // merging those inside the decode kernel saves the merge pass; with more CTAs than requests
  // splitting is the rule, and the dedicated pass merges faster than the in-kernel contraction,
  // which adds a device-scope store / count / reload round trip to every split item's tail.
  // A function of the parameters only, like every launch shape of a run.
  P.dec_contraction = p.contraction ? p.contraction : (p.num_ctas <= p.batch ? 1 : 2);

  // Levels: every item gets a state block of T_q rows (rows numbered level by level), except
  // write-through level items, which write their rows' final output.
  PlanScratch& X = plan_scratch();
  if ((int32_t)X.lv.size() < num_levels) X.lv.resize(num_levels);
  std::vector<Stage>& lv = X.lv;
  std::vector<int32_t>& flags = X.flags;   // 1: the request's output is written by one item
  flags.assign(B, 0);
  int32_t row = 0;
  for (int32_t l = 0; l < num_levels; ++l) {
    const pkc_level_host& h = levels[l];
    std::vector<int32_t>& qo = X.qo;
    qo.resize(h.num_groups);
    for (int32_t g = 0; g < h.num_groups; ++g) qo[g] = h.qo_indptr[g + 1] - h.qo_indptr[g];
    if ((s = lpt_plan(qo.data(), h.kv_lens, h.num_groups, p.level_tile_q, p.level_ctas, p.alpha,
                      p.beta, r.p.chunk_align, p.enable_split != 0, &lv[l], h.causal != 0)) != PKC_OK)
      return s;
    P.lvl_groups[l] = h.num_groups;
    P.lvl_causal[l] = h.causal != 0 ? 1 : 0;
    P.lvl_tile_q[l] = p.level_tile_q;
    P.lvl_items[l] = (int32_t)lv[l].items.size();
    P.lvl_kv_chunk[l] = lv[l].kv_chunk;
    P.lvl_row_base[l] = row;
    // Write-through candidates: groups none of whose requests has own KV, when this is the
    // plan's only level; among their items, those whose tile has a single chunk.
    std::vector<char>& wt_group = X.wt_group;
    wt_group.assign(h.num_groups, 0);
    if (p.level_write_through && num_levels == 1) {
      for (int32_t g = 0; g < h.num_groups; ++g) {
        bool own = false;
        for (int32_t b = h.qo_indptr[g]; b < h.qo_indptr[g + 1]; ++b) own = own || kv_lens_h[b] > 0;
        wt_group[g] = own ? 0 : 1;
      }
    }
    // Chunks per tile: the items of one tile are consecutive in w order.
    std::vector<int32_t>& chunks_of = X.chunks_of;
    chunks_of.assign(lv[l].items.size(), 0);
    for (size_t i = 0; i < lv[l].items.size();) {
      size_t j = i;
      while (j < lv[l].items.size() && lv[l].items[j].req == lv[l].items[i].req &&
             lv[l].items[j].tile == lv[l].items[i].tile)
        ++j;
      for (size_t k = i; k < j; ++k) chunks_of[k] = (int32_t)(j - i);
      i = j;
    }
    for (size_t i = 0; i < lv[l].items.size(); ++i) {
      Item& it = lv[l].items[i];
      it.q0 += h.qo_indptr[it.req];
      if (wt_group[it.req] && chunks_of[i] == 1) {
        it.row = -1;
        for (int32_t q = 0; q < it.nq; ++q) flags[it.q0 + q] = 1;
        ++P.lvl_write_through;
      } else {
        it.row = row;
        row += p.level_tile_q;
      }
    }
  }
  // Decode stage over every request's own KV (one query per request, T_q = 1).
  Stage& dec = X.dec;
  if ((s = lpt_plan(nullptr, kv_lens_h, B, 1, p.num_ctas, p.alpha, p.beta, r.p.chunk_align,
                    p.enable_split != 0, &dec)) != PKC_OK)
    return s;
  std::vector<int32_t>& chunks = X.chunks;
  chunks.assign(B, 0);
  for (const Item& it : dec.items) chunks[it.req]++;
  P.dec_row_base = row;
  int32_t slots = 0;
  // A request whose own KV is a single chunk is finished by that chunk's workgroup: it folds
  // in the request's level states (its merge list) and writes the final output.
  for (Item& it : dec.items) {
    it.q0 = it.req;
    if (chunks[it.req] == 1) {
      it.row = -1;
      flags[it.req] = 1;
    } else {
      it.row = row + slots++;
    }
  }
  row += slots;
  P.dec_items = (int32_t)dec.items.size();
  // Waves per decode workgroup (its waves split an item's pages): a launch shape, so it comes
  // from the parameters only and stays the same for every plan of one workspace.
  P.dec_waves = p.decode_waves ? p.decode_waves : 4;
  P.dec_slots = slots;
  P.dec_kv_chunk = dec.kv_chunk;
  P.state_rows = row;
  if (P.dec_items > L.max_dec_items || slots > L.max_dec_rows)
    return fail(PKC_ERR_INTERNAL, "decode stage exceeds its bound");
  for (int32_t l = 0; l < num_levels; ++l)
    if (P.lvl_items[l] > L.max_lvl_items[l]) return fail(PKC_ERR_INTERNAL, "level exceeds its bound");

  // Write stage arrays: indptr over CTAs, items in CTA-major assignment order.
  auto write_stage = [&](const Stage& st, int64_t off_indptr, int64_t off_items) {
    int32_t* indptr = reinterpret_cast<int32_t*>(base + off_indptr);
    Item* items = reinterpret_cast<Item*>(base + off_items);
    int32_t k = 0;
    indptr[0] = 0;
    for (int32_t c = 0; c < st.ctas; ++c) {
      for (int32_t w : st.cta[c]) items[k++] = st.items[w];
      indptr[c + 1] = k;
    }
  };
  for (int32_t l = 0; l < num_levels; ++l) write_stage(lv[l], L.off_lvl_indptr[l], L.off_lvl_items[l]);
  write_stage(dec, L.off_dec_indptr, L.off_dec_items);

  // Merge lists: per request, levels ascending (chunks ascending), then its own KV.
  const int32_t NL2 = num_levels + 2;
  int32_t* mptr = reinterpret_cast<int32_t*>(base + L.off_merge_ptr);
  int32_t* mrows = reinterpret_cast<int32_t*>(base + L.off_merge_rows);
  // Items listed by w are already (group, tile, chunk) ordered; bucket them per request.
  std::vector<std::vector<int32_t>>& per_req_lvl = X.per_req_lvl;
  const size_t nlists = (size_t)B * (num_levels + 1);
  if (per_req_lvl.size() < nlists) per_req_lvl.resize(nlists);
  for (size_t i = 0; i < nlists; ++i) per_req_lvl[i].clear();
  for (int32_t l = 0; l < num_levels; ++l)
    for (const Item& it : lv[l].items)
      if (it.row >= 0)
        for (int32_t q = 0; q < it.nq; ++q)
          per_req_lvl[(size_t)(it.q0 + q) * (num_levels + 1) + l].push_back(it.row + q);
  for (const Item& it : dec.items)
    if (it.row >= 0) per_req_lvl[(size_t)it.req * (num_levels + 1) + num_levels].push_back(it.row);
  int32_t* rlev = reinterpret_cast<int32_t*>(base + L.off_req_levels);
  int32_t n = 0, num_merge = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t l = 0; l <= num_levels; ++l) {
      mptr[b * NL2 + l] = n;
      const std::vector<int32_t>& rows_bl = per_req_lvl[(size_t)b * (num_levels + 1) + l];
      if (l < num_levels) {
        // The decode kernel computes a request's level rows as first + c * T_q (the chunks of
        // one query tile hold consecutive slots); keep that invariant checked.
        for (size_t c = 1; c < rows_bl.size(); ++c)
          if (rows_bl[c] != rows_bl[0] + (int32_t)c * p.level_tile_q)
            return fail(PKC_ERR_INTERNAL, "level rows of a request are not one query tile's chunks");
        rlev[(b * num_levels + l) * 2] = rows_bl.empty() ? 0 : rows_bl[0];
        rlev[(b * num_levels + l) * 2 + 1] = (int32_t)rows_bl.size();
      }
      for (int32_t rr : rows_bl) mrows[n++] = rr;
    }
    mptr[b * NL2 + num_levels + 1] = n;
    if (!flags[b]) ++num_merge;
  }
  if (n > L.max_merge_rows) return fail(PKC_ERR_INTERNAL, "merge list exceeds its bound");
  std::memcpy(base + L.off_req_flags, flags.data(), (size_t)B * 4);
  P.merge_entries = n;
  P.num_merge = num_merge;

  P.off_dec_indptr = L.off_dec_indptr;
  P.off_dec_items = L.off_dec_items;
  for (int32_t l = 0; l < num_levels; ++l) {
    P.off_lvl_indptr[l] = L.off_lvl_indptr[l];
    P.off_lvl_items[l] = L.off_lvl_items[l];
  }
  P.off_merge_ptr = L.off_merge_ptr;
  P.off_merge_rows = L.off_merge_rows;
  P.off_req_flags = L.off_req_flags;
  P.off_req_levels = L.off_req_levels;
  P.off_counters = L.off_counters;
  P.int_bytes = L.int_bytes;
  P.off_state_o = L.off_state_o;
  P.off_state_lse = L.off_state_lse;
  P.dev_bytes = L.dev_bytes;
  P.dev_ws = 0;
  *out = P;
  return PKC_OK;
}

}  // namespace pkc

extern "C" pkc_status pkc_plan_host(const pkc_plan_params* params, const int32_t* kv_lens_h,
                                    const pkc_level_host* levels_h, int32_t num_levels,
                                    void* host_buf, size_t host_bytes, pkc_plan_info* out) {
  try {
    pkc::clear_error();
    pkc::Resolved r;
    pkc_status s = pkc::check_params(params, true, &r);
    if (s != PKC_OK) return s;
    return pkc::build_plan_host(r, kv_lens_h, levels_h, num_levels, host_buf, host_bytes, out);
  } catch (...) {
    return pkc::fail(PKC_ERR_INTERNAL, "exception in pkc_plan_host");
  }
}

extern "C" pkc_status pkc_validate_block_table(const int32_t* block_table, int32_t max_blocks,
                                               const int32_t* cache_seqlens,
                                               const int32_t* kv_start, int32_t batch,
                                               int32_t page_size, int64_t num_pages) {
  try {
    pkc::clear_error();
    if (batch < 0 || max_blocks < 0 || page_size <= 0 || num_pages < 0)
      return pkc::fail(PKC_ERR_INVALID_ARG, "bad sizes");
    if (batch > 0 && (!block_table || !cache_seqlens))
      return pkc::fail(PKC_ERR_INVALID_ARG, "NULL array");
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t lo = kv_start ? kv_start[b] : 0, hi = cache_seqlens[b];
      if (lo < 0 || hi < lo)
        return pkc::fail(PKC_ERR_INVALID_ARG, "request " + std::to_string(b) + ": bad token range");
      if (hi == lo) continue;
      if ((hi - 1) / page_size >= max_blocks)
        return pkc::fail(PKC_ERR_INVALID_ARG, "request " + std::to_string(b) + ": length exceeds max_blocks * page_size");
      for (int64_t j = lo / page_size; j <= (hi - 1) / page_size; ++j) {
        const int32_t pg = block_table[(int64_t)b * max_blocks + j];
        if (pg < 0 || pg >= num_pages)
          return pkc::fail(PKC_ERR_INVALID_ARG, "request " + std::to_string(b) + ", block " +
                                                    std::to_string(j) + ": invalid page " + std::to_string(pg));
      }
    }
    return PKC_OK;
  } catch (...) {
    return pkc::fail(PKC_ERR_INTERNAL, "exception in pkc_validate_block_table");
  }
}
