// Paged batch-decode / suffix kernel for gfx950 (vector ALU, wave64): the kernel template and
// its launch helpers, instantiated by decode.hip (fp32 / fp16 / bf16 pools) and decode_fp8.hip
// (OCP FP8 E4M3 pools with fp16 / bf16 queries).
//
// Single-query attention ("Cascade Inference" blog, section on multi-query vs single-query
// kernels): every query has its own KV, so the work is bound by HBM reads of K and V and runs
// on the vector ALUs; no matrix cores.  Grouped-query heads that share a KV head are fused
// into one workgroup so each K/V row is read once for the whole group (FlashInfer paper
// summary, appendix A, head-group fusion).
//
// Mapping (D = 128, 16-bit types): a token row of one KV head is 256 contiguous bytes (head_dim
// contiguous, paper summary section A3 on data movement), read by 16 lanes with one 128-bit
// load each, so a wave64 load instruction covers 4 token rows; the q.k partial dot products are
// reduced inside each 16-lane DPP row without LDS.  Each 16-lane row keeps its own online-softmax
// state (running max m, sum l, accumulator), in base 2; the rows of a wave and the waves of a
// workgroup are combined at the end with the merge operator.  Pages come from the block table
// ("Paged attention" page, decode path).  Tokens outside the item's range and pages outside
// [0, num_pages) are never read: when a page holds whole 4-row loads, each load goes through a
// buffer resource over its page and masked lanes fall outside its range (the hardware returns
// zeros); with smaller pages masked lanes read row 0 of page 0 and select zeros.
//
// Each wave walks its steps as a software pipeline: while step s is computed, the K/V loads of
// step s+1 are in flight and the block-table entries of step s+2 are being fetched.  Table
// entries, plan records and other wave-uniform metadata go through the scalar cache, and every
// path issues the same number of vector loads, so waiting for step s never waits for s+1.
//
// A workgroup that finishes a request (its only chunk) also folds in the request's cascade
// level states.  A tile's chunks hold consecutive slots, so the request's rows at a level are
// first + c * T_q: each lane prefetches its share into registers at item start (a fixed number
// of buffer loads, empty ones outside the range) and writes it to LDS after its steps.
//
// Attention and contraction in one launch (FlashInfer paper summary, section A3: the partial
// outputs of split KV are contracted by the same persistent kernel, whose grid is fixed by the
// parameters).  Each workgroup that writes a partial state of a split request writes it with
// device-scope atomic stores (coherent across the XCDs' L2 caches without flushing them), waits
// for them to complete and then bumps the request's arrival counter (a device-scope atomic);
// the one that brings it to the request's number of partial states reads the request's states
// with device-scope atomic loads, merges its whole merge list (levels, then its own chunks)
// into the final output with the merge pass's arithmetic, and sets the counter back to zero.
// Nothing waits for another workgroup, so any number of workgroups may be resident.  Requests
// with no decode item and no write-through (empty KV; a cascade request with no own KV) are
// merged at the start of workgroup (b mod #CTA, kv head).
#pragma once

#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "merge_ops.h"

namespace pkc {

// K (and V) loads per lane per wave step of the decode kernel.
template <typename T, int G> struct DecodeLoads {
  static constexpr int kU = IsKV8<T>::value ? (G >= 4 ? 1 : 2) : (G >= 4 ? 2 : 4);
};

// PM (page mode): 0 = pages smaller than one load's token rows (page per lane); 1 = a page
// holds whole loads (page per sub-tile, wave-uniform); 2 = a page holds whole steps (one
// page per step).  FOLD: items that finish a request fold in its level states.
template <typename T, int D, int G, int NW, int PM, bool FOLD>
__global__ __launch_bounds__(64 * NW) void decode_kernel(const DecodeParams p) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int VEC = 16 / ES;        // elements per lane per load
  constexpr int LANES = D / VEC;      // lanes per token row
  constexpr int ROWS = 64 / LANES;    // token rows per wave load
  // Loads of K (and of V) per lane per step; with two steps in flight this is 8 (G <= 2) or
  // 4 (G >= 4, whose G accumulators already need the registers) outstanding K/V loads.  FP8
  // pools hold 16 elements per lane load (twice the accumulators), so half as many.
  constexpr int U = DecodeLoads<T, G>::kU;
  constexpr int TI = ROWS * U;        // tokens per wave step
  constexpr int CPROW = G * D / 4;    // 16-byte chunks of one state row (all G heads)
  static_assert(LANES >= 4 && LANES <= 32, "row width");

  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  // Level states of a finishing item, prefetched in FL 16-byte chunks per lane (O rows, dense,
  // level after level) plus one LSE value per lane.
  constexpr int FL = !FOLD ? 0 : (NW == 1 ? 4 : 8 / NW);
  constexpr int FCAP = FL * 64 * NW;   // chunk capacity
  __shared__ f4_t sm_fold[FOLD ? FCAP : 1];
  __shared__ float sm_fold_lse[FOLD ? 64 * NW : 1];
  __shared__ int sm_last;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LANES;
  const int col = lane % LANES;
  const int hk = blockIdx.y;
  const int hq0 = hk * G;
  const int shift = p.page_shift;
  const int P = p.page_size;
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  const int64_t head_off = (int64_t)hk * (D * ES) + col * 16;
  const int64_t slot_stride = (int64_t)p.hkv * (D * ES);
  // One page is under 2 GiB (checked on the host): offsets inside it fit in 32 bits.
  const int32_t head_off32 = (int32_t)head_off;
  const int32_t slot_stride32 = (int32_t)slot_stride;
  const int32_t page_bytes = P * slot_stride32;

  // Merge of request b's list rows [beg, end) for this workgroup's G heads into its output.
  using TO = typename OutType<T>::type;
  auto contract = [&](auto coherent, int b, int beg, int end) {
    for (int idx = threadIdx.x; idx < G * D / 4; idx += 64 * NW)
      merge_rows_to_output<TO, D, decltype(coherent)::value>(p.st_o, p.st_lse, p.merge_rows, beg, end, p.hq, b,
                                                              hq0 + idx / (D / 4), (idx % (D / 4)) * 4, p.o,
                                                              p.lse);
  };
  const int nlv = p.nl2 - 2;
  if (p.counters) {
    for (int b = blockIdx.x; b < p.batch; b += gridDim.x) {
      const int32_t* mp = p.merge_ptr + (int64_t)b * p.nl2;
      if (scalar_load(p.req_flags + b) == 0 && scalar_load(mp + nlv) == scalar_load(mp + nlv + 1))
        contract(std::false_type(), b, scalar_load(mp), scalar_load(mp + nlv + 1));
    }
  }

  int it_begin = 0, it_end = 1;
  if (p.indptr) {
    it_begin = scalar_load(p.indptr + blockIdx.x);
    it_end = scalar_load(p.indptr + blockIdx.x + 1);
  }
  for (int it = it_begin; it < it_end; ++it) {
    int b, tb, te, srow;
    if (p.indptr) {
      const int32_t* rec = p.items + 8 * (int64_t)it;
      b = scalar_load(rec);
      const int base = p.kv_start ? scalar_load(p.kv_start + b) : 0;
      tb = base + scalar_load(rec + 3);
      te = base + scalar_load(rec + 4);
      srow = scalar_load(rec + 5);
    } else {
      b = blockIdx.x;
      tb = p.kv_start ? scalar_load(p.kv_start + b) : 0;
      te = scalar_load(p.seqlens + b);
      srow = -1;
    }
    tb = max(tb, 0);
    te = min(te, p.max_blocks << shift);
    const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
    const int32_t* mptr = p.merge_ptr ? p.merge_ptr + (int64_t)b * p.nl2 : nullptr;

    QSlice<T> qv[G];   // the q elements matching this lane's K/V elements
#pragma unroll
    for (int j = 0; j < G; ++j)
      qv[j] = load_qslice<T>(static_cast<const char*>(p.q) + (((int64_t)b * p.hq + hq0 + j) * D) * QBytes<T>::kBytes, col);

    // Level states this item folds in when it finishes its request: level l holds cnt_l rows
    // first_l + c * T_q ({first_l, cnt_l} from the plan's per-request table), stored densely
    // from chunk cofs[l] (and LSE slot lofs[l]).  Up to MAXF levels are prefetched when they
    // fit; otherwise they are read directly at the end.  The scalar reads go out here; the
    // vector loads follow the first K/V loads (fold_issue).
    constexpr int MAXF = PKC_MAX_LEVELS < 4 ? PKC_MAX_LEVELS : 4;
    bool fold_reg = false;
    int nlev = 0;
    int cofs[MAXF + 1] = {}, lofs[MAXF + 1] = {}, first[MAXF] = {};
    f4_t fr[FL > 0 ? FL : 1];
    float flse = 0.f;
    if constexpr (FOLD) {
      if (srow < 0 && mptr && p.num_levels <= MAXF) {
        nlev = p.num_levels;
        // All MAXF entries are read at once (the table has 2 * MAXF ints of padding after it);
        // entries past the request's levels count as empty.
        const int32_t* rl = p.req_levels + (int64_t)b * nlev * 2;
        int ent[2 * MAXF];
#pragma unroll
        for (int k = 0; k < 2 * MAXF; ++k) ent[k] = scalar_load(rl + k);
#pragma unroll
        for (int l = 0; l < MAXF; ++l) {
          first[l] = ent[2 * l];
          const int cnt = l < nlev ? ent[2 * l + 1] : 0;
          cofs[l + 1] = cofs[l] + cnt * CPROW;
          lofs[l + 1] = lofs[l] + cnt * G;
        }
        fold_reg = p.fold_o_bytes > 0 && cofs[nlev] <= FCAP && lofs[nlev] <= 64 * NW;
      }
    }
    // Lane gl owns chunks f * 64 * NW + gl and LSE slot gl; each resolves to its level by
    // comparing with the (uniform) level boundaries.  Outside the range: empty loads.
    auto fold_issue = [&]() {
      if constexpr (FOLD) {
        const int gl = wv * 64 + lane;
        const rsrc_t ro = make_rsrc(p.st_o, fold_reg ? p.fold_o_bytes : 0);
        const rsrc_t rl = make_rsrc(p.st_lse, fold_reg ? p.fold_lse_bytes : 0);
#pragma unroll
        for (int f = 0; f < FL; ++f) {
          const int q = f * 64 * NW + gl;
          int32_t off = kOffsetNone;
#pragma unroll
          for (int l = 0; l < MAXF; ++l) {
            if (l < nlev && q >= cofs[l] && q < cofs[l + 1]) {
              const int c = (q - cofs[l]) / CPROW, rem = (q - cofs[l]) % CPROW;
              off = ((first[l] + c * p.lvl_tile_q[l]) * p.hq + hq0) * (D * 4) + rem * 16;
            }
          }
          const V16 x = buffer_load16(ro, off);
          fr[f] = f4_t{__uint_as_float(x.w[0]), __uint_as_float(x.w[1]), __uint_as_float(x.w[2]),
                       __uint_as_float(x.w[3])};
        }
        int32_t off = kOffsetNone;
#pragma unroll
        for (int l = 0; l < MAXF; ++l) {
          if (l < nlev && gl >= lofs[l] && gl < lofs[l + 1]) {
            const int c = (gl - lofs[l]) / G, j = (gl - lofs[l]) % G;
            off = ((first[l] + c * p.lvl_tile_q[l]) * p.hq + hq0 + j) * 4;
          }
        }
        flse = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, off, 0, 0));
      }
    };

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = kNegInf;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] = 0.f;
    }

    // Steps of this wave: token blocks blk0 + s*NW, s = 0 .. nsteps-1 (TI tokens each).
    const int blk0 = te > tb ? tb / TI + wv : 0;
    const int blk1 = te > tb ? (te - 1) / TI : -1;
    const int nsteps = blk0 <= blk1 ? (blk1 - blk0) / NW + 1 : 0;

    // Block-table entries of a step's U sub-tiles plus, in pg[U], the mask of sub-tiles inside
    // the range.  Branch-free: a sub-tile outside the range reads entry 0 of the row (it exists
    // whenever there are steps); entries are only examined when the step is issued, so the
    // scalar loads are not waited for here.
    auto fetch_pages = [&](int s, int (&pg)[U + 1]) {
#pragma unroll
      for (int i = 0; i <= U; ++i) pg[i] = 0;
      if constexpr (PM > 0) {
        const int tblk = (blk0 + s * NW) * TI;
        int need_mask = 0;
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const int tsub = tblk + i * ROWS;
          const bool need = (s < nsteps) & (tsub < te) & (tsub + ROWS > tb);
          need_mask |= (need ? 1 : 0) << i;
          if constexpr (PM == 1) pg[i] = scalar_load(bt + (need ? (tsub >> shift) : 0));
        }
        if constexpr (PM == 2) {
          // The step's TI tokens are TI-aligned and the page size is a multiple of TI.
          const int e = scalar_load(bt + (need_mask ? (tblk >> shift) : 0));
#pragma unroll
          for (int i = 0; i < U; ++i) pg[i] = e;
        }
        pg[U] = need_mask;
      }
    };
    // Issue the K/V loads of step s; bit i of ok marks a valid row of sub-tile i.  A step past
    // the wave's last one issues loads that return zeros (no sub-tile is inside the range).
    auto issue = [&](int s, const int (&pg)[U + 1], V16 (&kr)[U], V16 (&vr)[U], uint32_t& ok) {
      ok = 0;
      const int tblk = (blk0 + s * NW) * TI;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int t = tblk + i * ROWS + row;
        if constexpr (PM > 0) {
          // One page per sub-tile: a buffer over that page; rows outside [tb, te) and invalid
          // pages read past the buffer's range and come back as zeros.
          const bool pv = ((pg[U] >> i) & 1) & (pg[i] >= 0) & (pg[i] < p.num_pages);
          const bool v = pv & (t >= tb) & (t < te);
          ok |= (v ? 1u : 0u) << i;
          const int64_t pofs = pv ? (int64_t)pg[i] * page_bytes : 0;
          const rsrc_t rk = make_rsrc(kbase + pofs, pv ? page_bytes : 0);
          const rsrc_t rv = make_rsrc(vbase + pofs, pv ? page_bytes : 0);
          const int32_t off = v ? (t & (P - 1)) * slot_stride32 + head_off32 : kOffsetNone;
          kr[i] = buffer_load16<kCachePolicyStream>(rk, off);
          vr[i] = buffer_load16<kCachePolicyStream>(rv, off);
        } else {
          bool v = (t >= tb) && (t < te);
          const int page = v ? bt[t >> shift] : -1;
          v = v && page >= 0 && page < p.num_pages;
          ok |= (v ? 1u : 0u) << i;
          const int64_t off = (((int64_t)page << shift) + (t & (P - 1))) * slot_stride + head_off;
          kr[i] = load16_or_zero(kbase, off, v);
          vr[i] = load16_or_zero(vbase, off, v);
        }
      }
    };
    auto compute = [&](const V16 (&kr)[U], const V16 (&vr)[U], uint32_t ok) {
      float s[U][G];
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int j = 0; j < G; ++j) s[i][j] = dot16(T(), qv[j], kr[i]);
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float r = group_sum<LANES>(s[i][j]);
          s[i][j] = ((ok >> i) & 1u) ? r * p.scale_log2 : kNegInf;
        }
      float vf[U][VEC];
#pragma unroll
      for (int i = 0; i < U; ++i) unpack16(T(), vr[i], vf[i]);
      float mu[G], a[G];
      bool moved = false;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float mx = s[0][j];
#pragma unroll
        for (int i = 1; i < U; ++i) mx = fmaxf(mx, s[i][j]);
        const float mn = fmaxf(m[j], mx);
        mu[j] = (mn == kNegInf) ? 0.f : mn;
        a[j] = fast_exp2(m[j] - mu[j]);
        moved |= a[j] != 1.f;
        m[j] = mn;
      }
      // Once the running maxima settle no row rescales: one wave vote skips it for all heads.
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          l[j] *= a[j];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] *= a[j];
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const float pr = fast_exp2(s[i][j] - mu[j]);
          l[j] += pr;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pr, vf[i][e], acc[j][e]);
        }
      }
    };

    if (nsteps == 0) fold_issue();
    if (nsteps > 0) {
      int pgA[U + 1], pgB[U + 1];   // U table entries + mask of the sub-tiles that need them
      V16 kA[U], vA[U], kB[U], vB[U];
      uint32_t okA = 0, okB = 0;
      fetch_pages(0, pgA);
      fetch_pages(1, pgB);
      issue(0, pgA, kA, vA, okA);
      fold_issue();
      // Steps go in pairs (A, B) with the next step's loads always issued before the current
      // step is computed; a step past the end issues loads that return zeros.  Every path
      // then has the same loads in flight, so waiting for one step never waits for the next.
      // A scheduling barrier after each issue keeps the compiler from pulling the previous
      // step's arithmetic (which waits for its data) above the next step's loads.
      int s = 0;
      // Table entries for step s+2 are fetched after step s+1's loads: scalar loads return out
      // of order, so any wait for one waits for all, and these have a whole step to arrive.
      for (; s + 1 < nsteps; s += 2) {
        issue(s + 1, pgB, kB, vB, okB);
        __builtin_amdgcn_sched_barrier(0);
        fetch_pages(s + 2, pgA);
        __builtin_amdgcn_sched_barrier(0);
        compute(kA, vA, okA);
        issue(s + 2, pgA, kA, vA, okA);
        __builtin_amdgcn_sched_barrier(0);
        fetch_pages(s + 3, pgB);
        __builtin_amdgcn_sched_barrier(0);
        compute(kB, vB, okB);
      }
      if (s < nsteps) compute(kA, vA, okA);   // odd step count: the last step is in A
    }

    // Merge the ROWS row states of the wave (butterfly over lane offsets LANES .. 32).
#pragma unroll
    for (int off = LANES; off < 64; off <<= 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float m2 = __shfl_xor(m[j], off);
        const float l2 = __shfl_xor(l[j], off);
        float a2[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) a2[e] = __shfl_xor(acc[j][e], off);
        merge_state2<VEC>(m[j], l[j], acc[j], m2, l2, a2);
      }
    }

    // Merge the NW wave states through LDS (and, for a finishing request, its level states)
    // and write the item's state.
    if (row == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_acc[wv][j][col * VEC + e] = acc[j][e] * p.v_scale;
        if (col == 0) {
          sm_m[wv][j] = m[j];
          sm_l[wv][j] = l[j];
        }
      }
    }
    if constexpr (FOLD) {
      const int gl = wv * 64 + lane;
#pragma unroll
      for (int f = 0; f < FL; ++f) sm_fold[f * 64 * NW + gl] = fr[f];
      sm_fold_lse[gl] = flse;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
      const int j = idx / D, d = idx % D;
      const int h = hq0 + j;
      // Running merge in base 2: (mx, num, den) with num, den scaled by 2^-mx.
      float mx = kNegInf, num = 0.f, den = 0.f;
      auto absorb = [&](float s2, float o_val, float l_val) {
        const float mn = fmaxf(mx, s2);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float f0 = fast_exp2(mx - mu), f1 = fast_exp2(s2 - mu);
        num = num * f0 + o_val * f1;
        den = den * f0 + l_val * f1;
        mx = mn;
      };
      if (fold_reg) {
        const float* fo = reinterpret_cast<const float*>(sm_fold);
#pragma unroll
        for (int lv = 0; lv < MAXF; ++lv) {
          if (lv >= nlev) break;
          const int cnt = (lofs[lv + 1] - lofs[lv]) / G;
          for (int c = 0; c < cnt; ++c)
            absorb(sm_fold_lse[lofs[lv] + c * G + j] * kLog2e, fo[cofs[lv] * 4 + (c * G + j) * D + d], 1.f);
        }
      } else if (FOLD && srow < 0 && mptr) {
        // Level states that did not fit in LDS come straight from global memory.
        const int m0 = scalar_load(mptr), m1 = scalar_load(mptr + p.num_levels);
        for (int k = m0; k < m1; ++k) {
          const int64_t r = scalar_load(p.merge_rows + k);
          absorb(p.st_lse[r * p.hq + h] * kLog2e, p.st_o[(r * p.hq + h) * D + d], 1.f);
        }
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) absorb(sm_m[w][j], sm_acc[w][j][d], sm_l[w][j]);
      const float o = den > 0.f ? num / den : 0.f;
      const float lse = den > 0.f ? (mx + log2f(den)) * kLn2 : kNegInf;
      if (srow < 0) {
        Elem<typename OutType<T>::type>::store(p.o, ((int64_t)b * p.hq + h) * D + d, o);
        if (d == 0) p.lse[(int64_t)b * p.hq + h] = lse;
      } else if (p.counters) {
        // Read by the request's last workgroup while this kernel runs: coherent stores.
        __hip_atomic_store(p.st_o + ((int64_t)srow * p.hq + h) * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) __hip_atomic_store(p.st_lse + (int64_t)srow * p.hq + h, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        p.st_o[((int64_t)srow * p.hq + h) * D + d] = o;
        if (d == 0) p.st_lse[(int64_t)srow * p.hq + h] = lse;
      }
    }
    if (p.counters && srow >= 0) {
      // This workgroup's partial state is complete at device scope once its stores have
      // completed; then count it in.  The last arrival merges.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int32_t* mp = p.merge_ptr + (int64_t)b * p.nl2;
      if (threadIdx.x == 0) {
        const uint32_t expect = (uint32_t)(scalar_load(mp + nlv + 1) - scalar_load(mp + nlv));
        uint32_t* ctr = p.counters + (int64_t)b * p.hkv + hk;
        const bool last = atomicAdd(ctr, 1u) + 1u == expect;
        if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = last ? 1 : 0;
      }
      __syncthreads();
      if (sm_last) contract(std::true_type(), b, scalar_load(mp), scalar_load(mp + nlv + 1));
    }
    // Drain this item's stores before the next item's loads: with stores and loads both in
    // flight the compiler can no longer count loads in order and waits for all of them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

template <typename T, int D, int G, int NW, int PM>
inline hipError_t launch_decode_t(const DecodeParams& p, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, p.hkv), block(64 * NW);
  if constexpr (std::is_same<T, F32>::value) {
    // Cascades need the matrix-core prefix kernel, which takes 16-bit and FP8 pools only.
    if (p.num_levels > 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_kernel<T, D, G, NW, PM, false>), grid, block, 0, s, p);
  } else {
    if (p.num_levels > 0)
      hipLaunchKernelGGL((decode_kernel<T, D, G, NW, PM, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((decode_kernel<T, D, G, NW, PM, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <typename T, int D, int G, int NW>
inline hipError_t launch_decode_u(const DecodeParams& p, int grid_x, hipStream_t s) {
  constexpr int ROWS = 64 / (D / (16 / Elem<T>::kBytes));
  constexpr int TI = ROWS * DecodeLoads<T, G>::kU;   // tokens per wave step, as in the kernel
  if (p.page_size >= TI) return launch_decode_t<T, D, G, NW, 2>(p, grid_x, s);
  if (p.page_size >= ROWS) return launch_decode_t<T, D, G, NW, 1>(p, grid_x, s);
  return launch_decode_t<T, D, G, NW, 0>(p, grid_x, s);
}

template <typename T, int D, int G>
inline hipError_t launch_decode_w(int waves, const DecodeParams& p, int grid_x, hipStream_t s) {
  switch (waves) {
    case 1: return launch_decode_u<T, D, G, 1>(p, grid_x, s);
    case 2: return launch_decode_u<T, D, G, 2>(p, grid_x, s);
    default: return launch_decode_u<T, D, G, 4>(p, grid_x, s);
  }
}

template <typename T, int D>
inline hipError_t launch_decode_g(int group, int waves, const DecodeParams& p, int grid_x,
                                  hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_w<T, D, 1>(waves, p, grid_x, s);
    case 2: return launch_decode_w<T, D, 2>(waves, p, grid_x, s);
    case 4: return launch_decode_w<T, D, 4>(waves, p, grid_x, s);
    case 8: return launch_decode_w<T, D, 8>(waves, p, grid_x, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
inline hipError_t launch_decode_d(int head_dim, int group, int waves, const DecodeParams& p,
                                  int grid_x, hipStream_t s) {
  if (head_dim == 64) return launch_decode_g<T, 64>(group, waves, p, grid_x, s);
  if (head_dim == 128) return launch_decode_g<T, 128>(group, waves, p, grid_x, s);
  return hipErrorInvalidValue;
}

}  // namespace pkc
