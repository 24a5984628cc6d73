// Internal launch interface between the C ABI (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkc.h"

namespace pkc {

// Decode / suffix stage.  One workgroup per (CTA or request, KV head).
struct DecodeParams {
  const void* q;             // [B, Hq, D]
  const void* k;             // [num_pages, P, Hkv, D]
  const void* v;
  int64_t num_pages;
  const int32_t* block_table;  // [B, max_blocks]
  int32_t max_blocks;
  const int32_t* seqlens;    // [B] (plan == nullptr only)
  const int32_t* kv_start;   // [B] or nullptr
  int32_t hq, hkv, page_size, page_shift;
  float scale_log2;          // sm_scale * log2(e) (times the K scale for FP8 pools)
  float v_scale;             // V scale of FP8 pools (1 otherwise)
  void* o;                   // [B, Hq, D] dtype
  float* lse;                // [B, Hq]
  float* st_o;               // partial states [rows, Hq, D] fp32
  float* st_lse;             // [rows, Hq] natural-log LSE
  const int32_t* indptr;     // plan stage indptr [#CTA + 1] or nullptr (one item per request)
  const int32_t* items;      // plan items, 8 int32 each
  // Level states a finishing item folds in: merge_rows[merge_ptr[b*nl2] .. merge_ptr[b*nl2 +
  // num_levels]) (merge_ptr == nullptr: none).  At level l the rows of one request are
  // first + c * lvl_tile_q[l], c = 0, 1, ... (consecutive chunks of one query tile).
  const int32_t* merge_ptr;
  const int32_t* merge_rows;
  int32_t nl2, num_levels;
  int32_t lvl_tile_q[PKC_MAX_LEVELS];
  const int32_t* req_levels;  // [B, num_levels, 2] {first row, count} per request and level
  // Bytes of st_o / st_lse a finishing item may prefetch level states from through 32-bit
  // buffer offsets (0: states beyond 2 GiB, read directly at the end instead).
  int32_t fold_o_bytes, fold_lse_bytes;
  // In-kernel contraction (counters != nullptr; needs merge_ptr / merge_rows, nl2 = levels + 2):
  // the workgroup whose partial state of a split request arrives last merges the request's
  // merge list into its output, and a request with no decode item that no item writes through
  // (req_flags[b] == 0) is merged by workgroup (b mod #CTA, kv head).  counters [B, Hkv] are
  // zero before the launch and left zero by it.
  uint32_t* counters;
  const int32_t* req_flags;
  int32_t batch;
};

// Multi-query (MFMA) stage of one cascade level.
struct PrefixParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t num_pages;
  const int32_t* page_indptr;   // [G+1]
  const int32_t* page_indices;  // [nnz]
  int32_t num_page_indices;
  int32_t hq, hkv, page_size, page_shift;
  float scale_log2;             // sm_scale * log2(e) (times the K scale for FP8 pools)
  float v_scale;                // FP8 pools: V scale applied to the state (unused otherwise)
  float* st_o;
  float* st_lse;
  const int32_t* indptr;        // [#CTA + 1]
  const int32_t* items;
  // Ragged multi-token queries: page_indptr == nullptr selects a dense block table (group g's
  // pages are page_indices[g * table_stride ..]); the causal kernel variant masks query i of
  // group g (its queries are rows grp_qo_indptr[g] ..) to tokens t <= grp_kv_lens[g] - l_q(g) + i.
  const int32_t* grp_qo_indptr;
  const int32_t* grp_kv_lens;
  int32_t table_stride;
  // Items with state row -1 (level write-through, batch prefill) write their query rows' final
  // output here instead: O [rows, hq, D] in the operand type, LSE [rows, hq] fp32.
  void* o;
  float* lse;
  // Tree masks (causal variant only; nullptr: none): group g's mask is the l_q x l_q byte
  // matrix at tree_mask + mask_indptr[g] (row = query, column = new token, nonzero = visible),
  // inside a buffer of mask_bytes bytes.
  const uint8_t* tree_mask;
  const int32_t* mask_indptr;
  int32_t mask_bytes;
  // Deferred plan (plan_host != nullptr): the plan's integer words are still only in the
  // page-locked host buffer plan_host; this launch reads its items there and copies all
  // plan_words words to plan_dev (the workspace) for the launches that follow on the stream.
  // indptr and items keep their workspace addresses (their offsets locate the host copies).
  const int32_t* plan_host;
  int32_t* plan_dev;
  int32_t plan_words;
};

// Plan-driven merge: request b merges merge_rows[merge_ptr[b*NL2 + l0] .. merge_ptr[b*NL2 + l1]).
struct MergePlanParams {
  const float* st_o;
  const float* st_lse;
  const int32_t* merge_ptr;
  const int32_t* merge_rows;
  const int32_t* req_flags;  // skip requests with flag 1 (nullptr: never skip)
  int32_t nl2, l0, l1;
  int32_t batch, hq;
  void* o;
  float* lse;
};

struct MergeGenericParams {
  const void* o_states;
  const float* lse_states;
  int32_t num_states;
  const int32_t* indptr;
  const int32_t* indices;
  int32_t num_outputs, states_per_output, num_heads;
  void* o_out;
  float* lse_out;
};

// In-place KV append: request b's new K and V rows (row_bytes = Hkv * D * esize each, at
// k_new + b * row_bytes) go to slot seqlens[b] % P of page block_table[b][seqlens[b] / P].
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t page_shift;
  const int32_t* seqlens;
  int32_t* seqlens_out;      // nullable; may alias seqlens
  int64_t row_bytes;         // multiple of 16
};

// Multi-token append: request b's rows new_indptr[b] .. new_indptr[b+1]-1 of k_new / v_new.
struct AppendRaggedParams {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t page_shift;
  const int32_t* seqlens;
  const int32_t* new_indptr;   // [B+1]
  int64_t total_new;           // rows of k_new / v_new
  int32_t* seqlens_out;        // nullable; never aliases seqlens
  int64_t row_bytes;           // multiple of 16
};

hipError_t launch_decode(pkc_dtype dt, int head_dim, int group, int waves, const DecodeParams& p,
                         int grid_x, hipStream_t s);
// OCP FP8 E4M3 pools; q_dt (fp16 or bf16) is the type of q and o.
hipError_t launch_decode_fp8(pkc_dtype q_dt, int head_dim, int group, int waves,
                             const DecodeParams& p, int grid_x, hipStream_t s);
// streams: 1 = 4-wave workgroups (two per compute unit), 2 = 8-wave workgroups whose two
// 4-wave halves take alternate tiles of an item and merge at its end (one per compute unit).
hipError_t launch_prefix(pkc_dtype dt, int head_dim, int group, int tile_q, int streams,
                         const PrefixParams& p, int grid_x, hipStream_t s);
// The level kernel with the causal mask (ragged multi-token queries, fp16 / bf16 pools).
hipError_t launch_prefill_causal(pkc_dtype dt, int head_dim, int group, int tile_q, int streams,
                                 const PrefixParams& p, int grid_x, hipStream_t s);
hipError_t launch_prefill_causal_fp8(pkc_dtype q_dt, int head_dim, int group, int tile_q, int streams,
                                     const PrefixParams& p, int grid_x, hipStream_t s);
// The same over OCP FP8 E4M3 pools; q_dt (fp16 or bf16) is the query and operand type.
hipError_t launch_prefix_fp8(pkc_dtype q_dt, int head_dim, int group, int tile_q, int streams,
                             const PrefixParams& p, int grid_x, hipStream_t s);
hipError_t launch_merge_plan(pkc_dtype out_dt, int head_dim, const MergePlanParams& p,
                             hipStream_t s);
hipError_t launch_merge_generic(pkc_dtype in_dt, pkc_dtype out_dt, int head_dim,
                                const MergeGenericParams& p, hipStream_t s);
hipError_t launch_merge_inplace(pkc_dtype dt, int head_dim, void* o_a, float* lse_a,
                                const void* o_b, const float* lse_b, int64_t num_states,
                                hipStream_t s);
// Copies `bytes` (a multiple of 16, 16-byte aligned) from pinned host memory to the device.
hipError_t launch_plan_upload(const void* host_src, void* dev_dst, int64_t bytes, hipStream_t s);
hipError_t launch_append_kv(const AppendParams& p, int32_t batch, hipStream_t s);
hipError_t launch_append_kv_ragged(const AppendRaggedParams& p, int32_t batch, hipStream_t s);
// Reads `mib` MiB of src (16-byte aligned) once as a nontemporal stream; sink gets mib * 256
// uint32 values.
hipError_t launch_read_stream(const void* src, int64_t mib, uint32_t* sink, hipStream_t s);
hipError_t launch_debug_gather(const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seqlens, const int32_t* kv_start, int32_t batch,
                               int32_t page_shift, int64_t num_pages, int32_t* rows_out,
                               int32_t max_tokens, hipStream_t s);
hipError_t launch_debug_trace(const int32_t* indptr, const int32_t* items, int32_t ctas,
                              int32_t* trace_out, int32_t max_items_per_cta, hipStream_t s);

// Physical row (page * P + slot) of token t through a page list, or -1 (shared by the decode
// kernel's address computation and the gather debug export).
__device__ __forceinline__ int64_t token_row(const int32_t* pages, int32_t t, int32_t page_shift,
                                             int64_t num_pages) {
  const int32_t pg = pages[t >> page_shift];
  if (pg < 0 || pg >= num_pages) return -1;
  return ((int64_t)pg << page_shift) + (t & ((1 << page_shift) - 1));
}

}  // namespace pkc
