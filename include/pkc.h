/*
 * pkc.h -- C ABI of libpkc: paged-KV cascade decode attention for AMD MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Decode attention of one query token per request over a paged KV cache, returned as an
 * attention state: the output O and the log-sum-exp LSE of the scaled scores (natural log).
 * States of disjoint token sets of the same query combine with the merge operator
 *     (O, LSE)(I u J) = ( (e^{LSE_I} O_I + e^{LSE_J} O_J) / (e^{LSE_I} + e^{LSE_J}),
 *                         log(e^{LSE_I} + e^{LSE_J}) )
 * which is commutative and associative ("Attention States and Recursive Attention",
 * FlashInfer tutorial, merge operator equations; FlashInfer paper summary, section A2
 * "Attention composition").  Three uses of it are built in:
 *   - split-KV: a request's KV is cut into chunks that run on different workgroups and are
 *     merged in a second pass (the tutorial's "KV sequence parallelism" application);
 *   - cascade: queries that share a prefix attend to it with a multi-query (MFMA) kernel that
 *     reads the shared KV once, attend to their own suffix with the decode kernel, and the
 *     states are merged ("Cascade Inference" blog, algorithm section); more than two levels
 *     and several shared prefixes per level are supported (same blog, future-work section);
 *   - a CPU load-balancing plan assigns KV chunks to workgroups (FlashInfer paper summary,
 *     section A3, "load-balancing scheduling"; appendix D, workspace and write-through).
 *
 * Data layout (all device arrays are caller-owned, contiguous, row-major)
 * ---------------------------------------------------------------------
 *   q            [B, Hq, D]                 dtype      one query token per request
 *   k_pool,v_pool[num_pages, P, Hkv, D]     dtype      head_dim contiguous; token t of a page
 *                                                      run lives in page run[t / P], slot t % P
 *   block_table  [B, max_blocks]            int32      physical page of each logical block of a
 *                                                      request; -1 = not allocated ("Paged
 *                                                      attention" page, decode path)
 *   cache_seqlens[B]                        int32      cached tokens per request
 *   o            [B, Hq, D]                 out dtype  final output (rounded once, RNE)
 *   lse          [B, Hq]                    float32    natural-log LSE; -inf for an empty set
 * Query head h reads KV head h / (Hq / Hkv) (grouped-query attention, contiguous groups).
 * A request attends over exactly the tokens [kv_start[b], cache_seqlens[b]) of its table
 * row: blocks past the last cached token are never dereferenced, so a block allocated for the
 * next token (or -1) there is harmless.  An invalid entry (-1 or >= num_pages) INSIDE that
 * range is a caller error: the kernels never read memory through it (such a page contributes
 * no tokens) and pkc_validate_block_table reports it.
 *
 * Supported: dtype f32 / f16 / bf16 (q, k, v share it); head_dim 64 or 128; page size a power
 * of two in [1, 1024] with one page (page_size x Hkv x head_dim elements) under 2 GiB;
 * Hq / Hkv in {1, 2, 4, 8}.  The multi-query prefix kernel needs f16 or bf16 and page size
 * >= 4; other combinations return PKC_ERR_UNSUPPORTED.
 *
 * Conventions
 * -----------
 * Every function is extern "C", never throws, and returns a pkc_status.  On failure
 * pkc_last_error() gives a thread-local message.  All shape/argument checks happen on the host
 * before any launch.  Device work is enqueued on the caller's HIP stream (`stream`, a
 * hipStream_t; NULL = the null stream) and calls return without synchronising.  The library
 * never allocates or frees device or pinned memory; the plan and the partial states live in a
 * caller-provided device workspace whose size pkc_plan_buffer_sizes returns.  The only global
 * state is cached device properties and the optional timing ring (pkc_timing_*); no
 * environment variable is read.
 */
#ifndef PKC_H
#define PKC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkc_status {
  PKC_OK = 0,
  PKC_ERR_INVALID_ARG = 1,         /* bad pointer, shape, length or parameter */
  PKC_ERR_UNSUPPORTED = 2,         /* dtype / head_dim / page size / group size not built */
  PKC_ERR_WORKSPACE_TOO_SMALL = 3, /* host or device buffer smaller than required */
  PKC_ERR_PLAN_MISMATCH = 4,       /* plan built for other shapes or another workspace */
  PKC_ERR_HIP = 5,                 /* a HIP runtime call failed (message has the HIP error) */
  PKC_ERR_INTERNAL = 6
} pkc_status;

typedef enum pkc_dtype { PKC_F32 = 0, PKC_F16 = 1, PKC_BF16 = 2 } pkc_dtype;

#define PKC_MAX_LEVELS 8
#define PKC_PLAN_MAGIC 0x504b4331u /* "PKC1" */

/* Diagnostics. */
const char* pkc_status_string(pkc_status s);
const char* pkc_last_error(void);
const char* pkc_version(void);

/* sizeof of the ABI structs below, so that language bindings can check their mirrors. */
void pkc_abi_struct_sizes(size_t* plan_params, size_t* level_host, size_t* level_dev,
                          size_t* plan_info);

/* Compute units and wavefront size of a device (HIP device ordinal). */
pkc_status pkc_device_info(int32_t device, int32_t* num_cus, int32_t* wave_size,
                           int64_t* lds_bytes_per_block);

/*
 * Plan parameters.  The plan follows the load-balancing scheduler of the FlashInfer paper
 * summary (section A3): the cost of a tile is alpha * l_q + beta * l_kv; the maximum chunk is
 * L_kv = ceil(sum_i ceil(l_qo(i) / T_q) * l_kv(i) / #CTA) (rounded up to chunk_align); every
 * tile's KV is cut greedily into chunks of at most L_kv; chunks are sorted longest first
 * (stable) and each goes to the CTA with the smallest cost so far (ties: smaller CTA index).
 * A CTA is one workgroup per KV head (head-group fusion, paper appendix A): a stage launches
 * #CTA x Hkv workgroups.
 */
typedef struct pkc_plan_params {
  int32_t batch;        /* B: requests (one query token each) */
  int32_t num_qo_heads; /* Hq */
  int32_t num_kv_heads; /* Hkv (divides Hq) */
  int32_t head_dim;     /* D */
  int32_t page_size;    /* P */
  int32_t num_ctas;     /* #CTA of the decode stage; 0 -> max(ceil(8 x compute units / Hkv),
                           batch): about 8 workgroups per compute unit, at least one CTA per
                           request */
  int32_t level_ctas;   /* #CTA of every cascade level; 0 -> max(1, floor(compute units / Hkv)) */
  int32_t level_tile_q; /* T_q of the cascade levels (queries per tile); 0 -> 128 / (Hq/Hkv) */
  int32_t chunk_align;  /* round L_kv up to a multiple of this; 0 or 1 -> no rounding */
  int32_t enable_split; /* 0 -> L_kv = longest KV length (one chunk per tile, no split-KV) */
  int64_t alpha;        /* cost per query row (>= 0) */
  int64_t beta;         /* cost per KV token (>= 0) */
  int32_t decode_waves; /* waves per decode workgroup: 0 -> 4; 1, 2 or 4.  Short items (a few
                           dozen tokens) run faster on 1 or 2 waves.  Like every launch shape of a
                           run, it depends on the parameters only, never on the lengths of a step,
                           so one run captured in a HIP graph stays valid for every plan built
                           from the same parameters into the same workspace */
  int32_t level_write_through; /* 1 (batch prefill): in a plan with a single level, a tile of a
                           group whose requests have no own KV and whose KV is one chunk writes its
                           rows' final output (O in the query type, LSE) instead of a state, and
                           the merge pass skips those rows; only pkc_batch_prefill_paged(_fp8)
                           runs such plans.  0: every level item writes a state (cascades) */
  int32_t level_streams; /* tile streams per level workgroup: 0 -> 2 when level_ctas x Hkv is at
                           most the compute-unit count (one 8-wave workgroup per compute unit,
                           two 4-wave streams over alternate KV tiles, merged at the end), else
                           1 (4-wave workgroups); 1 or 2 fix it */
  int32_t contraction;  /* where the partial states of split requests are merged (the
                           contraction of the FlashInfer paper summary, section A3):
                           1 -> inside the decode kernel (attention and contraction in one
                           launch: the workgroup whose partial state of a request arrives last
                           merges that request's states; requests with no decode item are
                           merged by the decode workgroups too), so a decode or cascade run
                           launches no merge pass; 2 -> a separate merge pass after the decode
                           kernel; 0 -> 1 when num_ctas <= batch (few split requests), else 2.
                           Both give the same bits. */
  int32_t defer_upload; /* 0: pkc_plan enqueues the copy of the plan into the workspace.
                           1: pkc_plan enqueues nothing; the plan stays in host_buf (which must
                           then be page-locked) and the first run call that uses it brings it
                           over: in pkc_cascade_decode(_fp8) with levels, the first level kernel
                           reads its own items from host_buf and copies the plan into the
                           workspace while it runs (no separate launch); every other run call
                           enqueues the copy first.  host_buf must then stay untouched until
                           the run calls that use the plan have completed on their stream.
                           Same results either way. */
} pkc_plan_params;

/* Host description of one cascade level: groups of consecutive requests sharing a KV run.
 * Group g holds requests qo_indptr[g] <= b < qo_indptr[g+1] (0 <= qo_indptr[0],
 * non-decreasing, qo_indptr[G] <= B) and attends over kv_lens[g] tokens.  causal != 0 (ragged
 * multi-token queries, pkc_batch_prefill_paged with causal): group g's requests are the last
 * l = qo_indptr[g+1] - qo_indptr[g] tokens of its sequence, so a query tile whose last query is
 * the i-th of the group (0-based) needs only tokens [0, kv_lens[g] - l + i + 1); the plan
 * chunks and weighs that extent instead of kv_lens[g]. */
typedef struct pkc_level_host {
  int32_t num_groups;
  const int32_t* qo_indptr; /* [G+1] host */
  const int32_t* kv_lens;   /* [G] host, tokens */
  int32_t causal;
} pkc_level_host;

/* Device description of one cascade level (block-sparse row view of the KV cache, paper
 * summary section A3): token t of group g is in page kv_page_indices[kv_page_indptr[g] + t/P],
 * slot t % P.  The group's run must hold ceil(kv_lens[g] / P) pages. */
typedef struct pkc_level_dev {
  const int32_t* kv_page_indptr;  /* [G+1] device */
  const int32_t* kv_page_indices; /* [nnz] device */
  int32_t num_page_indices;       /* nnz: the kernel clamps every group's run into the list */
} pkc_level_dev;

/*
 * A plan: plain data describing where the plan's integer arrays and the partial states sit in
 * the device workspace.  Produced by pkc_plan / pkc_plan_host, consumed by the run calls.
 * The integer arrays are laid out identically in the host buffer and the device workspace
 * (see pkc_plan for the format).  Do not edit; a plan is valid only with the workspace it was
 * built for.
 */
typedef struct pkc_plan_info {
  uint32_t magic;
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, page_size;
  int32_t num_levels;
  int32_t num_ctas;        /* decode stage #CTA (resolved) */
  int32_t level_ctas;      /* level #CTA (resolved) */
  int32_t dec_items;       /* work items of the decode stage */
  int32_t dec_slots;       /* partial slots of the decode stage */
  int32_t dec_kv_chunk;    /* L_kv of the decode stage */
  int32_t dec_waves;       /* waves per decode workgroup (1, 2 or 4), from the parameters */
  int32_t lvl_groups[PKC_MAX_LEVELS];
  int32_t lvl_tile_q[PKC_MAX_LEVELS];
  int32_t lvl_items[PKC_MAX_LEVELS];
  int32_t lvl_kv_chunk[PKC_MAX_LEVELS];
  int32_t lvl_row_base[PKC_MAX_LEVELS]; /* first state row of each level */
  int32_t dec_row_base;    /* first state row of the decode stage */
  int32_t state_rows;      /* rows of the fp32 partial-state buffer */
  int32_t merge_entries;   /* length of the merge row list */
  int32_t num_merge;       /* requests merged from several states (by the decode kernel or the
                              merge pass, per dec_contraction) */
  int64_t off_dec_indptr;  /* byte offsets inside the host buffer / device workspace */
  int64_t off_dec_items;
  int64_t off_lvl_indptr[PKC_MAX_LEVELS];
  int64_t off_lvl_items[PKC_MAX_LEVELS];
  int64_t off_merge_ptr;
  int64_t off_merge_rows;
  int64_t off_req_flags;
  int64_t off_req_levels;
  int64_t int_bytes;       /* bytes of integer plan data (copied host -> device) */
  int64_t off_state_o;     /* fp32 [state_rows, Hq, D] */
  int64_t off_state_lse;   /* fp32 [state_rows, Hq] */
  int64_t dev_bytes;       /* device workspace bytes this plan uses */
  uint64_t dev_ws;         /* address of the workspace the plan was copied to (0: host-only) */
  int32_t lvl_causal[PKC_MAX_LEVELS]; /* 1: the level was planned with causal tile extents */
  int32_t lvl_write_through;  /* level items that write the final output (level_write_through) */
  int32_t lvl_streams;     /* tile streams per level workgroup (1 or 2), from the parameters */
  int32_t dec_contraction; /* 1: the decode kernel merges split requests (no merge pass);
                              2: a merge pass follows it; from the parameters */
  int64_t off_counters;    /* uint32 [B, Hkv] arrival counters of the in-kernel contraction:
                              zero in every plan's integer arrays, and every run leaves them
                              zero */
  uint64_t host_src;       /* defer_upload: the page-locked host buffer the run calls copy the
                              plan from (0: pkc_plan enqueued the copy) */
} pkc_plan_info;

/*
 * Upper bounds of the pinned host buffer and device workspace for any plan with these
 * parameters and level shapes (only num_groups and qo_indptr of each level are read;
 * kv_lens may be NULL), so that pointers can stay fixed across steps (paper appendix D: the
 * workspace is sized from upper bounds for graph capture).  The decode stage's partial
 * states are bounded by 2 x #CTA rows, the appendix-D bound 2 x #CTA x T_q x Hq x (D + 1)
 * floats with T_q = 1.
 */
pkc_status pkc_plan_buffer_sizes(const pkc_plan_params* params, const pkc_level_host* levels,
                                 int32_t num_levels, size_t* host_bytes, size_t* device_bytes);

/*
 * Build a plan on the CPU and enqueue its copy into the device workspace.  For a page-locked
 * host buffer the copy is a small kernel on `stream` that reads the buffer directly (no
 * copy-engine synchronisation between steps); other host memory goes through hipMemcpyAsync.
 *   kv_lens_h: [B] host, tokens each request attends over in its own KV (the suffix in a
 *              cascade; cache_seqlens - kv_start for a plain decode).
 *   levels_h:  num_levels cascade levels (0 for a plain split-KV decode).
 *   host_buf:  caller-owned pinned host buffer (hipHostMalloc / torch pin_memory) of at least
 *              the size pkc_plan_buffer_sizes returned; it must stay untouched until the copy
 *              enqueued on `stream` has completed.
 *   dev_ws:    caller-owned device workspace (256-byte aligned).
 * Plan format (int32 arrays at the plan's offsets):
 *   stage indptr [#CTA + 1]: items of CTA c are [indptr[c], indptr[c+1]), in assignment order;
 *   stage items  8 int32 per item: {group_or_request, first_query, num_queries, kv_begin,
 *                kv_end, state_row (-1 = written to the final output), tile, w};
 *   merge_ptr    [B, num_levels + 2]: the merge rows of request b for level l are
 *                merge_rows[merge_ptr[b][l] .. merge_ptr[b][l+1]) (level num_levels = the
 *                request's own KV), in merge order: levels ascending, chunks ascending;
 *   merge_rows   state rows; req_flags [B]: 1 when the decode stage writes the output (the
 *                request's own KV is a single chunk; that chunk's workgroup first folds in
 *                the request's level states listed in merge_rows), 0 when the merge kernel
 *                does;
 *   req_levels   [B, num_levels, 2]: {first state row, count} of request b's rows at level
 *                l; they are first + c * lvl_tile_q[l] for c < count (the chunks of one query
 *                tile hold consecutive slots), the same rows merge_rows lists; 8 ints of
 *                padding follow.
 */
pkc_status pkc_plan(const pkc_plan_params* params, const int32_t* kv_lens_h,
                    const pkc_level_host* levels_h, int32_t num_levels, void* host_buf,
                    size_t host_bytes, void* dev_ws, size_t dev_bytes, void* stream,
                    pkc_plan_info* out);

/* The same plan without any HIP call (for CPU-side checks): fills host_buf and *out only;
 * out->dev_ws is 0.  num_ctas / level_ctas must be given explicitly (no device query). */
pkc_status pkc_plan_host(const pkc_plan_params* params, const int32_t* kv_lens_h,
                         const pkc_level_host* levels_h, int32_t num_levels, void* host_buf,
                         size_t host_bytes, pkc_plan_info* out);

/*
 * Paged batch decode ("Paged attention" page, decode path; "Cascade Inference" blog,
 * single-query kernels): request b attends over tokens [kv_start[b], cache_seqlens[b]).
 *   plan == NULL: one workgroup per (request, KV head); every request writes o/lse directly.
 *   plan != NULL: split-KV over the plan's decode stage (kv_lens_h of the plan must equal
 *                 cache_seqlens - kv_start; the token ranges come from the plan); unsplit
 *                 requests write o/lse directly (write-through, paper appendix D), split ones
 *                 write fp32 partial states to the workspace and a merge kernel finishes them.
 *                 The plan must have no levels.
 *   kv_start: NULL = 0 for every request.
 * dev_ws / dev_bytes may be NULL / 0 when plan is NULL.
 */
pkc_status pkc_batch_decode_paged(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                  const void* v_pool, int64_t num_pages,
                                  const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* cache_seqlens, const int32_t* kv_start,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t page_size, pkc_dtype dtype,
                                  float sm_scale, void* o, float* lse, void* dev_ws,
                                  size_t dev_bytes, void* stream);

/*
 * Multi-query attention of one cascade level ("Cascade Inference" blog, algorithm step 1):
 * every request covered by the level attends over its group's KV run; the group's queries run
 * as the rows of MFMA tiles so the run is read from HBM once per tile, not once per request.
 * The level's chunks are computed per the plan and merged into o_state [B, Hq, D] (o_dtype)
 * and lse_state [B, Hq]; requests the level does not cover get the identity (0, -inf).
 */
pkc_status pkc_prefix_attention(const pkc_plan_info* plan, int32_t level, const void* q,
                                const void* k_pool, const void* v_pool, int64_t num_pages,
                                const pkc_level_dev* level_dev, int32_t batch,
                                int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t page_size, pkc_dtype dtype, float sm_scale,
                                void* o_state, pkc_dtype o_dtype, float* lse_state,
                                void* dev_ws, size_t dev_bytes, void* stream);

/*
 * n-ary merge of attention states ("Attention States and Recursive Attention", n-ary merge
 * equation; maximum subtracted for stability):
 *   o_states [num_states, H, D] (in_dtype), lse_states [num_states, H] fp32.
 *   Output i merges states indices[indptr[i] .. indptr[i+1]) in that order (indices NULL: the
 *   states indptr[i] .. indptr[i+1]); indptr NULL: states i*S .. i*S + S - 1 with
 *   S = states_per_output.  Zero states, or all LSE = -inf, give (0, -inf).
 *   o_out [num_outputs, H, D] (out_dtype), lse_out [num_outputs, H].
 * indptr / indices are device arrays and are not range-checked on the device beyond
 * 0 <= index < num_states (out-of-range indices are skipped).
 */
pkc_status pkc_merge_states(const void* o_states, pkc_dtype in_dtype, const float* lse_states,
                            int32_t num_states, const int32_t* indptr, const int32_t* indices,
                            int32_t num_outputs, int32_t states_per_output, int32_t num_heads,
                            int32_t head_dim, void* o_out, pkc_dtype out_dtype, float* lse_out,
                            void* stream);

/* Binary merge in place: (o_a, lse_a) <- (o_a, lse_a) merged with (o_b, lse_b), for
 * num_rows x num_heads states of head_dim; o_a and o_b share `dtype`. */
pkc_status pkc_merge_state_inplace(void* o_a, float* lse_a, const void* o_b, const float* lse_b,
                                   int32_t num_rows, int32_t num_heads, int32_t head_dim,
                                   pkc_dtype dtype, void* stream);

/*
 * Cascade decode ("Cascade Inference" blog, algorithm section, generalised to num_levels
 * levels): for every level, the multi-query kernel over each group's KV run; then the decode
 * kernel over every request's own KV (block_table rows, tokens [0, suffix_seqlens[b]) per the
 * plan); then one merge per request of all its states in the order levels ascending, chunks
 * ascending, own KV last.  The plan must have been built with the same levels and with
 * kv_lens_h == suffix_seqlens.  A request whose own KV is a single chunk is finished by the
 * decode kernel (which folds in its level states); the merge kernel finishes the others.
 * With a plan, every run call enqueues the same kernels with the same arguments for every plan
 * built from the same parameters and level shapes into the same workspace (the merge kernel is
 * always enqueued and skips the requests flagged as finished), so a run captured in a HIP graph
 * can be replayed after any later pkc_plan into that workspace (paper summary, section A3:
 * plan outside the graph, run inside it).
 */
pkc_status pkc_cascade_decode(const pkc_plan_info* plan, const void* q, const void* k_pool,
                              const void* v_pool, int64_t num_pages,
                              const pkc_level_dev* levels, int32_t num_levels,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* suffix_seqlens, int32_t batch, int32_t num_qo_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                              pkc_dtype dtype, float sm_scale, void* o, float* lse, void* dev_ws,
                              size_t dev_bytes, void* stream);

/*
 * Allocation-free split-KV batch decode, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation and kernels as pkc_batch_decode_paged with a plan, but the workspace is a fixed
 * device array inside the library (PKC_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the
 * library runs on until the process ends) instead of a caller-provided one; the call
 * allocates and frees nothing.
 *   plan:          a plan without levels built by pkc_plan_host (or pkc_plan: its workspace is
 *                  ignored) for these shapes; its integer arrays are in plan_host_buf
 *                  (plan_host_bytes >= plan->int_bytes).  The call enqueues their copy into the
 *                  array on `stream` before the kernels; a page-locked buffer is read by a
 *                  kernel and must stay untouched until that copy has run.
 *   other arguments: as pkc_batch_decode_paged.
 * Errors: PKC_ERR_WORKSPACE_TOO_SMALL when the plan needs more than PKC_NOALLOC_SCRATCH_BYTES of
 * workspace (plan->dev_bytes; decided before any HIP call), PKC_ERR_PLAN_MISMATCH for a plan
 * with levels or other shapes.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams or threads) race; calls on one stream run in order.
 */
#define PKC_NOALLOC_SCRATCH_BYTES (32u << 20)
pkc_status pkc_batch_decode_paged_noalloc(const pkc_plan_info* plan, const void* plan_host_buf,
                                          size_t plan_host_bytes, const void* q, const void* k_pool,
                                          const void* v_pool, int64_t num_pages,
                                          const int32_t* block_table, int32_t max_blocks,
                                          const int32_t* cache_seqlens, const int32_t* kv_start,
                                          int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t page_size, pkc_dtype dtype,
                                          float sm_scale, void* o, float* lse, void* stream);

/*
 * Paged batch decode over FP8 K/V pools (the FlashInfer paper summary, appendix F: KV in fp8
 * with fp16 queries and outputs).  The pools hold OCP FP8 E4M3 codes, one byte per element,
 * same layout [num_pages, P, Hkv, D]; element value = decoded code * k_scale (K) or * v_scale
 * (V), the scales being per-pool floats (> 0).  q is [B, Hq, D] of q_dtype (PKC_F16 or
 * PKC_BF16) and o is written in q_dtype; LSE and partial states are fp32 as in
 * pkc_batch_decode_paged, whose other arguments and rules this call shares (plan == NULL or a
 * plan without levels).
 */
pkc_status pkc_batch_decode_paged_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                      const void* v_pool, float k_scale, float v_scale,
                                      int64_t num_pages, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* cache_seqlens,
                                      const int32_t* kv_start, int32_t batch,
                                      int32_t num_qo_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                      float sm_scale, void* o, float* lse, void* dev_ws,
                                      size_t dev_bytes, void* stream);

/*
 * pkc_prefix_attention over FP8 K/V pools (paper summary, appendix F): the same call and rules
 * with OCP FP8 E4M3 pools (one byte per element, [num_pages, P, Hkv, D]) whose element values
 * are decoded code * k_scale (K) and * v_scale (V), per-pool floats > 0.  q_dtype (PKC_F16 or
 * PKC_BF16) is the type of q and of the matrix-core operands (every E4M3 value is exact in
 * both); o_state / lse_state are written as in pkc_prefix_attention.
 */
pkc_status pkc_prefix_attention_fp8(const pkc_plan_info* plan, int32_t level, const void* q,
                                    const void* k_pool, const void* v_pool, float k_scale,
                                    float v_scale, int64_t num_pages,
                                    const pkc_level_dev* level_dev, int32_t batch,
                                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t page_size, pkc_dtype q_dtype, float sm_scale,
                                    void* o_state, pkc_dtype o_dtype, float* lse_state,
                                    void* dev_ws, size_t dev_bytes, void* stream);

/*
 * pkc_cascade_decode over FP8 K/V pools (paper summary, appendix F, with the "Cascade
 * Inference" blog's algorithm): every level and every request's own KV are read from OCP FP8
 * E4M3 pools with per-pool scales k_scale and v_scale (> 0); q and o are q_dtype (PKC_F16 or
 * PKC_BF16), LSE and partial states fp32.  Arguments and rules are those of
 * pkc_cascade_decode.
 */
pkc_status pkc_cascade_decode_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                  const void* v_pool, float k_scale, float v_scale,
                                  int64_t num_pages, const pkc_level_dev* levels,
                                  int32_t num_levels, const int32_t* block_table,
                                  int32_t max_blocks, const int32_t* suffix_seqlens,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                  float sm_scale, void* o, float* lse, void* dev_ws,
                                  size_t dev_bytes, void* stream);

/*
 * Ragged multi-token queries over the paged KV cache (prefill / append attention): the
 * "Paged attention" page's varlen indexing (cu_seq_lens_q packing of queries without padding)
 * over the decode path's block tables, as the FlashInfer paper summary's ragged query tensors
 * over a block-sparse KV cache (section A3).  Request b (0 <= b < num_requests) owns query
 * rows qo_indptr[b] .. qo_indptr[b+1]-1 of q ([total_q, Hq, D], dtype PKC_F16 or PKC_BF16)
 * and attends over tokens [0, kv_lens[b]) of its block-table row (block_table [num_requests,
 * max_blocks], -1 = unallocated; the new tokens already appended).  Its l_q(b) queries are
 * the sequence's last tokens: with causal != 0, query i sees tokens t <= kv_lens[b] - l_q(b)
 * + i (none when negative); with causal == 0 it sees all kv_lens[b] tokens.  Writes o
 * ([total_q, Hq, D], q's dtype) and lse ([total_q, Hq], fp32, natural log, -inf for a query
 * that sees no token).
 * The plan must be built by pkc_plan with batch = total_q (each query row is one plan
 * request), kv_lens_h all zero, and one level whose num_groups = num_requests, qo_indptr =
 * the same qo_indptr (host copy) and kv_lens = the same kv_lens (host copy); the run is the
 * level's multi-query kernel (query tiles of T_q rows, KV chunks by the plan) followed by the
 * merge of every query row's chunk states.  qo_indptr and kv_lens here are device arrays.
 * Errors: PKC_ERR_PLAN_MISMATCH when the plan does not have that shape; PKC_ERR_UNSUPPORTED
 * for fp32 queries or page_size < 4.  Pointers are caller-owned; the work is enqueued on
 * `stream`.
 */
pkc_status pkc_batch_prefill_paged(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                   const void* v_pool, int64_t num_pages,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* qo_indptr, const int32_t* kv_lens,
                                   int32_t num_requests, int32_t total_q, int32_t num_qo_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                   pkc_dtype dtype, float sm_scale, int32_t causal, void* o,
                                   float* lse, void* dev_ws, size_t dev_bytes, void* stream);

/*
 * Tree (speculative) decoding over ragged queries: pkc_batch_prefill_paged with causal = 1 and
 * a logits mask (paper summary: tree decoding in speculative decoding, section A2; the
 * LogitsMask of the attention-variant functors, section A3).  Request b's mask is the
 * l_q x l_q byte matrix at tree_mask + mask_indptr[b] (l_q = qo_indptr[b+1] - qo_indptr[b];
 * row i = query i, column j = new token j, the request's last l_q KV tokens; nonzero =
 * visible).  Query i sees every token before the new ones and new token j where the byte is
 * set, within its causal limit (bytes above the diagonal are ignored).  tree_mask (mask_bytes
 * bytes) and mask_indptr ([num_requests]) are device buffers; bytes past mask_bytes read as 0.
 * The plan is a causal prefill plan; other arguments and rules are those of
 * pkc_batch_prefill_paged.
 */
pkc_status pkc_batch_prefill_paged_tree(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_pages,
                                        const int32_t* block_table, int32_t max_blocks,
                                        const int32_t* qo_indptr, const int32_t* kv_lens,
                                        const uint8_t* tree_mask, const int32_t* mask_indptr,
                                        int32_t mask_bytes, int32_t num_requests, int32_t total_q,
                                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t page_size, pkc_dtype dtype, float sm_scale, void* o,
                                        float* lse, void* dev_ws, size_t dev_bytes, void* stream);

/*
 * pkc_batch_prefill_paged over FP8 K/V pools (paper summary, appendix F): OCP FP8 E4M3 codes
 * with per-pool scales k_scale and v_scale (> 0); q and o are q_dtype (PKC_F16 or PKC_BF16).
 * Arguments, plan and rules are those of pkc_batch_prefill_paged.  With one query per request
 * this is also a batch decode whose grouped query heads go through the matrix cores.
 */
pkc_status pkc_batch_prefill_paged_fp8(const pkc_plan_info* plan, const void* q, const void* k_pool,
                                       const void* v_pool, float k_scale, float v_scale,
                                       int64_t num_pages, const int32_t* block_table,
                                       int32_t max_blocks, const int32_t* qo_indptr,
                                       const int32_t* kv_lens, int32_t num_requests,
                                       int32_t total_q, int32_t num_qo_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, pkc_dtype q_dtype,
                                       float sm_scale, int32_t causal, void* o, float* lse,
                                       void* dev_ws, size_t dev_bytes, void* stream);

/*
 * In-place KV append ("Paged attention" page, decode path: the cache is updated in place, and
 * its worked example places each sequence's next token at logical block cache_seqlens[b] / P,
 * slot cache_seqlens[b] % P of the sequence's block-table row).  For every request b, the new
 * token's rows k_new[b] and v_new[b] ([B, Hkv, D] each, the dtype of the pools) are copied to
 * row (block_table[b][cache_seqlens[b] / P], cache_seqlens[b] % P) of k_pool and v_pool
 * ([num_pages, P, Hkv, D]), and new_seqlens[b] = cache_seqlens[b] + 1 (new_seqlens may be
 * NULL, or alias cache_seqlens for an in-place update).  Decoding over new_seqlens then
 * attends over the appended token as well.
 * A target block outside the table row, unallocated (-1) or naming a page outside
 * [0, num_pages) is a caller error: nothing is written for that request and new_seqlens[b]
 * keeps the old length.  All pointers are device pointers owned by the caller; the work is
 * enqueued on `stream`.  Returns PKC_ERR_INVALID_ARG / PKC_ERR_UNSUPPORTED on bad sizes.
 */
pkc_status pkc_append_kv(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* cache_seqlens, int32_t* new_seqlens, int32_t batch,
                         int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                         pkc_dtype dtype, void* stream);

/*
 * Multi-token in-place append (the append / prefill path; "Paged attention" page, decode path:
 * the cache is updated in place at the next-token position of each sequence, applied here to
 * every new token in order).  Request b's new rows are k_new / v_new rows new_indptr[b] ..
 * new_indptr[b+1]-1 ([total_new, Hkv, D] each, the dtype of the pools); row new_indptr[b] + i
 * goes to row (block_table[b][(cache_seqlens[b] + i) / P], (cache_seqlens[b] + i) % P) of
 * k_pool and v_pool, and new_seqlens[b] = cache_seqlens[b] + n_b (n_b = new_indptr[b+1] -
 * new_indptr[b]); a prefill over new_seqlens then attends over the new tokens.  A request with
 * a missing target block (outside the row, -1, or a page outside [0, num_pages)), or with an
 * inconsistent row range (decreasing indptr, rows past total_new), is a caller error: nothing
 * is written for it and new_seqlens[b] keeps the old length.  new_seqlens may be NULL and must
 * not alias cache_seqlens.  new_indptr, cache_seqlens, new_seqlens and the tensors are device
 * pointers owned by the caller; the work is enqueued on `stream`.  Returns
 * PKC_ERR_INVALID_ARG / PKC_ERR_UNSUPPORTED on bad sizes, NULL pointers or aliasing.
 */
pkc_status pkc_append_kv_ragged(const void* k_new, const void* v_new, int64_t total_new,
                                const int32_t* new_indptr, void* k_pool, void* v_pool,
                                int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* cache_seqlens, int32_t* new_seqlens, int32_t batch,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                pkc_dtype dtype, void* stream);

/*
 * Host-side check of block-table contents (host arrays): every block holding one of the
 * tokens [kv_start[b], cache_seqlens[b]) must name a page in [0, num_pages).  Returns
 * PKC_ERR_INVALID_ARG naming the first bad (request, block) otherwise.  Not on the hot path.
 */
pkc_status pkc_validate_block_table(const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* cache_seqlens, const int32_t* kv_start,
                                    int32_t batch, int32_t page_size, int64_t num_pages);

/*
 * Debug export of the integer gather: rows_out[b * max_tokens + t] = the physical row
 * page * P + slot that the kernels read for token t (t < max_tokens) of request b, or -1
 * when t is outside [kv_start[b], cache_seqlens[b]) or its block entry is invalid.  Uses the
 * same device address routine as the decode kernel.
 */
pkc_status pkc_debug_gather_rows(const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* cache_seqlens, const int32_t* kv_start,
                                 int32_t batch, int32_t page_size, int64_t num_pages,
                                 int32_t* rows_out, int32_t max_tokens, void* stream);

/*
 * Debug export of the work-to-workgroup map as the device walks it: for stage `stage`
 * (0 .. num_levels-1 = a level, num_levels = the decode stage), workgroup c writes, for its
 * k-th item, the item's 8 plan fields to trace_out[(c * max_items_per_cta + k) * 8 ...];
 * unused entries are -1.  trace_len counts int32 elements.
 */
pkc_status pkc_debug_cta_trace(const pkc_plan_info* plan, int32_t stage, const void* dev_ws,
                               int32_t* trace_out, int64_t trace_len,
                               int32_t max_items_per_cta, void* stream);

/*
 * Measurement export: reads `bytes` bytes of device memory at `src` once, as a stream of
 * 16-byte nontemporal loads with 16 loads in flight per lane (the load form the attention
 * kernels use for K and V), so that its duration gives the device's achievable HBM read
 * rate.  `bytes` must be a positive multiple of 1 MiB and `src` 16-byte aligned; `sink`
 * (device, caller-owned) receives bytes / 1 MiB * 256 uint32 values (sink_len counts them).
 * Enqueued on `stream`; returns PKC_ERR_INVALID_ARG on bad sizes or alignment.
 */
pkc_status pkc_read_stream_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_len,
                                 void* stream);

/*
 * Per-kernel timing with HIP events (for measurements): when enabled, every kernel launch
 * of the calls above is bracketed by events recorded on the same stream (created without the
 * system-scope fence on record, so the brackets add no cache writeback between kernels).
 * Launches on a stream that is being captured into a graph are not bracketed (nor counted).
 * pkc_timing_read waits for the recorded events and returns, per kernel kind, the number of
 * launches and the summed duration in milliseconds since the last reset.
 * Kernel kinds: 0 decode, 1 prefix (MFMA), 2 merge (plan-driven), 3 merge (generic / in place).
 */
pkc_status pkc_timing_enable(int32_t enable);
pkc_status pkc_timing_reset(void);
pkc_status pkc_timing_read(int32_t kind, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* PKC_H */
