// Paged batch-decode / suffix kernel for gfx950 (vector ALU, wave64).
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
// ("Paged attention" page, decode path); the page index of a 4-row load is wave-uniform, so the
// table entry is a scalar load.  Tokens outside the item's range and pages outside
// [0, num_pages) are never read.
//
// Each wave walks its steps as a software pipeline: while step s is computed, the K/V loads of
// step s+1 are in flight and the block-table entries of step s+2 are being fetched, so neither
// the table read nor the KV read latency sits between two steps.
//
// A workgroup that finishes a request (its only chunk) also folds in the request's cascade
// level states listed in the plan's merge list, so the cascade needs no separate merge pass
// for such requests.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace pkc {

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(const DecodeParams p) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int VEC = 16 / ES;        // elements per lane per load
  constexpr int LANES = D / VEC;      // lanes per token row
  constexpr int ROWS = 64 / LANES;    // token rows per wave load
  // Loads of K (and of V) per lane per step; with two steps in flight this is 8 (G <= 2) or
  // 4 (G >= 4, whose G accumulators already need the registers) outstanding K/V loads.
  constexpr int U = G >= 4 ? 2 : 4;
  constexpr int TI = ROWS * U;        // tokens per wave step
  static_assert(LANES >= 4 && LANES <= 32, "row width");

  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  // Level states of a finishing item, prefetched straight into LDS (+ one load's slack).
  constexpr int kFoldFloats = 4096;
  __shared__ __attribute__((aligned(16))) float sm_fold[kFoldFloats + 256];
  __shared__ float sm_fold_lse[64];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LANES;
  const int col = lane % LANES;
  const int hk = blockIdx.y;
  const int hq0 = hk * G;
  const int shift = p.page_shift;
  const int P = p.page_size;
  const bool uniform_pages = P >= ROWS;  // a 4-row (ROWS-row) load never spans two pages
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  const int64_t head_off = (int64_t)hk * (D * ES) + col * 16;
  const int64_t slot_stride = (int64_t)p.hkv * (D * ES);

  int it_begin = 0, it_end = 1;
  if (p.indptr) {
    it_begin = p.indptr[blockIdx.x];
    it_end = p.indptr[blockIdx.x + 1];
  }
  for (int it = it_begin; it < it_end; ++it) {
    int b, tb, te, srow;
    if (p.indptr) {
      const int32_t* rec = p.items + 8 * (int64_t)it;
      b = rec[0];
      const int base = p.kv_start ? p.kv_start[b] : 0;
      tb = base + rec[3];
      te = base + rec[4];
      srow = rec[5];
    } else {
      b = blockIdx.x;
      tb = p.kv_start ? p.kv_start[b] : 0;
      te = p.seqlens[b];
      srow = -1;
    }
    tb = max(tb, 0);
    te = min(te, p.max_blocks << shift);
    const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;
    // Level states this item folds in when it finishes its request (read early; used at the end).
    int lv_beg = 0, lv_end = 0;
    if (srow < 0 && p.merge_ptr) {
      lv_beg = p.merge_ptr[(int64_t)b * p.nl2];
      lv_end = p.merge_ptr[(int64_t)b * p.nl2 + p.num_levels];
    }
    const int nfold = lv_end - lv_beg;
    const bool fold_lds = nfold > 0 && nfold * G * D <= kFoldFloats && nfold * G <= 64;
    // Direct global -> LDS loads of the level states (lane l of a load writes 16 bytes at
    // base + 16*l); they complete while the KV stream runs and are read back at the end.
    auto prefetch_fold = [&]() {
      if (!fold_lds) return;
      constexpr int CPRow = G * D / 4;   // 16-byte chunks per state row (all G heads)
      const int nchunks = nfold * CPRow;
      const int ninst = (nchunks + 63) / 64;
      for (int k = wv; k < ninst; k += NW) {
        const int q = min(k * 64 + lane, nchunks - 1);   // surplus lanes land in the slack
        const int64_t r = p.merge_rows[lv_beg + q / CPRow];
        const float* src = p.st_o + (r * p.hq + hq0) * D + (q % CPRow) * 4;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(sm_fold + k * 256),
                                         16, 0, 0);
      }
      if (wv == 0) {
        const int q = min(lane, nfold * G - 1);
        const int64_t r = p.merge_rows[lv_beg + q / G];
        __builtin_amdgcn_global_load_lds(p.st_lse + r * p.hq + hq0 + q % G,
                                         (__attribute__((address_space(3))) void*)sm_fold_lse, 4, 0, 0);
      }
    };

    V16 qv[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
      qv[j] = load16(static_cast<const char*>(p.q) + (((int64_t)b * p.hq + hq0 + j) * D) * ES + col * 16);

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

    // Block-table entries of a step's U sub-tiles (-1: sub-tile outside the range).
    auto fetch_pages = [&](int s, int (&pg)[U]) {
#pragma unroll
      for (int i = 0; i < U; ++i) pg[i] = -1;
      if (s < nsteps && uniform_pages) {
        const int tblk = (blk0 + s * NW) * TI;
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const int tsub = tblk + i * ROWS;
          if (tsub < te && tsub + ROWS > tb) pg[i] = bt[tsub >> shift];
        }
      }
    };
    // Issue the K/V loads of step s; bit i of ok marks a valid row of sub-tile i.
    auto issue = [&](int s, const int (&pg)[U], V16 (&kr)[U], V16 (&vr)[U], uint32_t& ok) {
      ok = 0;
      const int tblk = (blk0 + s * NW) * TI;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int t = tblk + i * ROWS + row;
        bool v = (t >= tb) && (t < te);
        int page = pg[i];
        if (!uniform_pages) page = v ? bt[t >> shift] : -1;
        v = v && page >= 0 && page < p.num_pages;
        ok |= (v ? 1u : 0u) << i;
        const int64_t off = (((int64_t)page << shift) + (t & (P - 1))) * slot_stride + head_off;
        kr[i] = v ? load16(kbase + off) : zero16();
        vr[i] = v ? load16(vbase + off) : zero16();
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
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float mx = s[0][j];
#pragma unroll
        for (int i = 1; i < U; ++i) mx = fmaxf(mx, s[i][j]);
        const float mn = fmaxf(m[j], mx);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float a = fast_exp2(m[j] - mu);
        m[j] = mn;
        l[j] *= a;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] *= a;
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const float pr = fast_exp2(s[i][j] - mu);
          l[j] += pr;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pr, vf[i][e], acc[j][e]);
        }
      }
    };

    if (nsteps == 0) prefetch_fold();
    if (nsteps > 0) {
      int pgA[U], pgB[U];
      V16 kA[U], vA[U], kB[U], vB[U];
      uint32_t okA = 0, okB = 0;
      fetch_pages(0, pgA);
      fetch_pages(1, pgB);
      issue(0, pgA, kA, vA, okA);
      prefetch_fold();
      for (int s = 0; s < nsteps; s += 2) {
        // Even step: compute A, B's loads in flight, pages of s+2 into pgA.
        fetch_pages(s + 2, pgA);
        if (s + 1 < nsteps) issue(s + 1, pgB, kB, vB, okB);
        compute(kA, vA, okA);
        if (s + 1 >= nsteps) break;
        // Odd step: compute B, A's loads in flight, pages of s+3 into pgB.
        fetch_pages(s + 3, pgB);
        if (s + 2 < nsteps) issue(s + 2, pgA, kA, vA, okA);
        compute(kB, vB, okB);
      }
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

    // Merge the NW wave states through LDS (and, for a finished request, its level states)
    // and write the item's state.
    if (row == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_acc[wv][j][col * VEC + e] = acc[j][e];
        if (col == 0) {
          sm_m[wv][j] = m[j];
          sm_l[wv][j] = l[j];
        }
      }
    }
    // The prefetched level states have landed in LDS once this wave's loads are done.
    if (fold_lds) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
      const int j = idx / D, d = idx % D;
      const int h = hq0 + j;
      // Running merge in base 2: (mx, num, den) with num, den scaled by 2^-mx.
      float mx = kNegInf, num = 0.f, den = 0.f;
      if (fold_lds) {
        float bm = kNegInf;
        for (int r = 0; r < nfold; ++r) bm = fmaxf(bm, sm_fold_lse[r * G + j]);
        bm *= kLog2e;
        const float mu = (bm == kNegInf) ? 0.f : bm;
        for (int r = 0; r < nfold; ++r) {
          const float f1 = fast_exp2(fmaf(sm_fold_lse[r * G + j], kLog2e, -mu));
          num = fmaf(sm_fold[(r * G + j) * D + d], f1, num);
          den += f1;
        }
        mx = bm;
      }
      // Otherwise level rows come from global memory, 16 at a time so their loads are in
      // flight together.
      constexpr int KB = 16;
      for (int k0 = fold_lds ? lv_end : lv_beg; k0 < lv_end; k0 += KB) {
        float sr[KB], orow[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          sr[u] = kNegInf;
          orow[u] = 0.f;
          if (k0 + u < lv_end) {
            const int64_t r = p.merge_rows[k0 + u];
            sr[u] = p.st_lse[r * p.hq + h] * kLog2e;
            orow[u] = p.st_o[(r * p.hq + h) * D + d];
          }
        }
        float bm = sr[0];
#pragma unroll
        for (int u = 1; u < KB; ++u) bm = fmaxf(bm, sr[u]);
        const float mn = fmaxf(mx, bm);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float f0 = fast_exp2(mx - mu);
        num *= f0;
        den *= f0;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const float f1 = fast_exp2(sr[u] - mu);
          num = fmaf(orow[u], f1, num);
          den += f1;
        }
        mx = mn;
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w][j];
        const float mn = fmaxf(mx, mw);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        const float f0 = fast_exp2(mx - mu), f1 = fast_exp2(mw - mu);
        num = num * f0 + sm_acc[w][j][d] * f1;
        den = den * f0 + sm_l[w][j] * f1;
        mx = mn;
      }
      const float o = den > 0.f ? num / den : 0.f;
      const float lse = den > 0.f ? (mx + log2f(den)) * kLn2 : kNegInf;
      if (srow < 0) {
        Elem<T>::store(p.o, ((int64_t)b * p.hq + h) * D + d, o);
        if (d == 0) p.lse[(int64_t)b * p.hq + h] = lse;
      } else {
        p.st_o[((int64_t)srow * p.hq + h) * D + d] = o;
        if (d == 0) p.st_lse[(int64_t)srow * p.hq + h] = lse;
      }
    }
    __syncthreads();
  }
}

// Waves per workgroup: the environment variable PKC_DECODE_WAVES (1, 2 or 4) overrides the
// choice made by the caller (used for tuning measurements).
static int env_waves() {
  static int w = [] {
    const char* s = std::getenv("PKC_DECODE_WAVES");
    const int v = s ? std::atoi(s) : 0;
    return (v == 1 || v == 2 || v == 4) ? v : 0;
  }();
  return w;
}

template <typename T, int D, int G, int NW>
static hipError_t launch_decode_t(const DecodeParams& p, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, p.hkv), block(64 * NW);
  hipLaunchKernelGGL((decode_kernel<T, D, G, NW>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_decode_w(int waves, const DecodeParams& p, int grid_x, hipStream_t s) {
  switch (waves) {
    case 1: return launch_decode_t<T, D, G, 1>(p, grid_x, s);
    case 2: return launch_decode_t<T, D, G, 2>(p, grid_x, s);
    default: return launch_decode_t<T, D, G, 4>(p, grid_x, s);
  }
}

template <typename T, int D>
static hipError_t launch_decode_g(int group, int waves, const DecodeParams& p, int grid_x,
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
static hipError_t launch_decode_d(int head_dim, int group, int waves, const DecodeParams& p,
                                  int grid_x, hipStream_t s) {
  if (head_dim == 64) return launch_decode_g<T, 64>(group, waves, p, grid_x, s);
  if (head_dim == 128) return launch_decode_g<T, 128>(group, waves, p, grid_x, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(pkc_dtype dt, int head_dim, int group, int waves, const DecodeParams& p,
                         int grid_x, hipStream_t s) {
  if (grid_x <= 0) return hipSuccess;
  if (env_waves()) waves = env_waves();
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
