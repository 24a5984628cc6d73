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
// ("Paged attention" page, decode path); the page index is wave-uniform, so the table entry is
// a scalar load.  Tokens outside the item's range and pages outside [0, num_pages) are never
// read.
#include "device_common.h"
#include "kernels.h"

namespace pkc {

constexpr int kDecodeWaves = 4;

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(const DecodeParams p) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int VEC = 16 / ES;        // elements per lane per load
  constexpr int LANES = D / VEC;      // lanes per token row
  constexpr int ROWS = 64 / LANES;    // token rows per wave load
  constexpr int U = 4;                // loads of K (and of V) in flight per lane per step
  constexpr int TI = ROWS * U;        // tokens per wave step
  static_assert(LANES >= 4 && LANES <= 32, "row width");

  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];

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

    if (te > tb) {
      const int blk0 = tb / TI, blk1 = (te - 1) / TI;
      for (int blk = blk0 + wv; blk <= blk1; blk += NW) {
        const int tblk = blk * TI;
        V16 kr[U], vr[U];
        bool ok[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
          const int tsub = tblk + i * ROWS;
          const int t = tsub + row;
          bool v = (t >= tb) && (t < te);
          int page;
          if (P >= ROWS) {
            // The whole sub-tile lies in one page: one scalar table read.
            page = (tsub < te && tsub + ROWS > tb) ? bt[tsub >> shift] : -1;
          } else {
            page = v ? bt[t >> shift] : -1;
          }
          v = v && page >= 0 && page < p.num_pages;
          ok[i] = v;
          const int64_t off =
              ((((int64_t)page << shift) + (t & (P - 1))) * p.hkv + hk) * (int64_t)(D * ES) + col * 16;
          kr[i] = v ? load16(kbase + off) : zero16();
          vr[i] = v ? load16(vbase + off) : zero16();
        }
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
            s[i][j] = ok[i] ? r * p.scale_log2 : kNegInf;
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

    // Merge the NW wave states through LDS and write the item's state.
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
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
      const int j = idx / D, d = idx % D;
      float mn = sm_m[0][j];
#pragma unroll
      for (int w = 1; w < NW; ++w) mn = fmaxf(mn, sm_m[w][j]);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(sm_m[w][j] - mu);
        num = fmaf(sm_acc[w][j][d], f, num);
        den = fmaf(sm_l[w][j], f, den);
      }
      const float o = den > 0.f ? num / den : 0.f;
      const float lse = den > 0.f ? (mu + log2f(den)) * kLn2 : kNegInf;
      const int h = hq0 + j;
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

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeParams& p, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, p.hkv), block(64 * kDecodeWaves);
  hipLaunchKernelGGL((decode_kernel<T, D, G, kDecodeWaves>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_g(int group, const DecodeParams& p, int grid_x, hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_t<T, D, 1>(p, grid_x, s);
    case 2: return launch_decode_t<T, D, 2>(p, grid_x, s);
    case 4: return launch_decode_t<T, D, 4>(p, grid_x, s);
    case 8: return launch_decode_t<T, D, 8>(p, grid_x, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_d(int head_dim, int group, const DecodeParams& p, int grid_x,
                                  hipStream_t s) {
  if (head_dim == 64) return launch_decode_g<T, 64>(group, p, grid_x, s);
  if (head_dim == 128) return launch_decode_g<T, 128>(group, p, grid_x, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(pkc_dtype dt, int head_dim, int group, const DecodeParams& p, int grid_x,
                         hipStream_t s) {
  if (grid_x <= 0) return hipSuccess;
  switch (dt) {
    case PKC_F32: return launch_decode_d<F32>(head_dim, group, p, grid_x, s);
    case PKC_F16: return launch_decode_d<F16>(head_dim, group, p, grid_x, s);
    case PKC_BF16: return launch_decode_d<BF16>(head_dim, group, p, grid_x, s);
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
