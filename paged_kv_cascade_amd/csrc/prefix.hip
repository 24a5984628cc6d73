// Multi-query attention over a shared KV run (one cascade level) for gfx950, on MFMA.
//
// "Cascade Inference" blog, algorithm step 1 and Fig. 3: the queries of all requests that
// share a prefix attend to it together, so the prefix KV is staged once on chip and reused by
// every query instead of being fetched once per request.  The FlashInfer paper summary
// (section A3, composable formats) describes the same thing as a dense block of the KV
// block-sparse matrix processed with a large row tile.  Many queries against one KV set is a
// real dense contraction, so both products run on matrix cores.
//
// Workgroup = 4 waves = 128 query rows (a row is one (query, head) pair of the KV head's
// group; heads of one query are adjacent rows).  Per 64-token KV tile:
//   * the 256 threads gather the tile's K and V rows (128-bit loads of head_dim-contiguous
//     rows, pages through the level's page list) into LDS, both row-major;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16} (tokens are the M dimension, so each lane
//     owns one query column and the softmax reductions are mostly in-lane);
//   * online softmax in base 2 (running max / sum per query);
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T accumulators, and V^T's
//     operand is read with the gfx950 LDS transpose read (ds_read_b64_tr_b16), which hands
//     each lane one head_dim column of four consecutive token rows.
// The tile loop is double buffered: the global loads of tile i+1 are in flight while tile i is
// computed, and the page ids of tile i+2 are fetched one iteration before they are needed.
// Output: one fp32 state (O normalised, natural-log LSE) per (query, head, item).
#include "device_common.h"
#include "kernels.h"

namespace pkc {

namespace {

constexpr int kTK = 64;        // KV tokens per tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kRowsPerWave = 32;

typedef short s4_t __attribute__((ext_vector_type(4)));

typedef float f2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even packing of two floats into the operand type is one gfx950
// instruction (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <typename T> struct Mfma;
template <> struct Mfma<F16> {
  __device__ static f4_t run(const V16& a, const V16& b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{lo, hi}, h2_t));
  }
};
template <> struct Mfma<BF16> {
  __device__ static f4_t run(const V16& a, const V16& b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{lo, hi}, b2_t));
  }
};

// True on every lane when `pred` holds on every active lane of the wave.
__device__ __forceinline__ bool wave_all(bool pred) {
  return __builtin_amdgcn_ballot_w64(!pred) == 0;
}

__device__ __forceinline__ V16 lds_load16(const char* p) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  V16 r;
  r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
  return r;
}

// Transpose read: within each 16-lane group, lanes 4i .. 4i+3 name the four 8-byte pieces of
// row i (16 consecutive 16-bit values); lane j of the group receives element j of rows 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  const s4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

}  // namespace

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads, 2) void prefix_kernel(const PrefixParams p) {
  constexpr int ES = 2;
  constexpr int STRIDE = D * ES + 16;          // bytes per K / V row in LDS (padded)
  constexpr int KBYTES = kTK * STRIDE;
  constexpr int BUF = 2 * KBYTES + kTK;        // K, V, one valid flag byte per token
  constexpr int CPR = D * ES / 16;             // 16-byte chunks per row
  constexpr int NPT = kTK * CPR / kThreads;    // tokens per loading thread (4 for D=128)
  constexpr int KS = D / 32;                   // contraction steps of S^T
  constexpr int DM = D / 16;                   // 16-row tiles of O^T
  static_assert(NPT == 2 || NPT == 4, "loader layout");

  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lg = lane >> 4;              // lane group 0..3
  const int hk = blockIdx.y;
  const int shift = p.page_shift;
  const int P = p.page_size;
  const char* kg = static_cast<const char*>(p.k);
  const char* vg = static_cast<const char*>(p.v);
  const int64_t row_stride = (int64_t)p.hkv * D * ES;   // bytes between consecutive slots
  // Loader role: chunk c of tokens tg*NPT .. tg*NPT+NPT-1 of the tile (one page: P >= NPT).
  const int ld_c = tid % CPR;
  const int ld_tg = tid / CPR;
  // Transpose-read role inside the lane group: row (4 tokens apart) and 8-byte column piece.
  const int tr_row = (lane & 15) >> 2;
  const int tr_piece = lane & 3;

  const int it_begin = p.indptr[blockIdx.x], it_end = p.indptr[blockIdx.x + 1];
  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* rec = p.items + 8 * (int64_t)it;
    const int grp = rec[0], q0 = rec[1], nq = rec[2], kb = rec[3], ke = rec[4], srow = rec[5];
    const int nrows = nq * G;
    const int32_t* pages = p.page_indices + p.page_indptr[grp];
    const int npages_grp = p.page_indptr[grp + 1] - p.page_indptr[grp];
    const int t0 = (kb / kTK) * kTK;
    const int ntiles = ke > kb ? (ke - t0 + kTK - 1) / kTK : 0;
    const bool wave_active = wv * kRowsPerWave < nrows;

    // Q^T operands: lane owns query row r = wv*32 + nt*16 + l16, head_dim slice
    // ks*32 + 8*lg .. +8 per contraction step.
    V16 qb[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = wv * kRowsPerWave + nt * 16 + l16;
      const bool ok = r < nrows;
      const int64_t qoff = ((int64_t)(q0 + r / G) * p.hq + hk * G + r % G) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[nt][ks] = ok ? load16(static_cast<const char*>(p.q) + (qoff + ks * 32 + 8 * lg) * ES) : zero16();
    }

    f4_t oacc[DM][2];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) oacc[dm][nt] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {kNegInf, kNegInf};
    float l_run[2] = {0.f, 0.f};

    // Page of this thread's token group in a tile (-1: no token of the group is in range).
    auto page_of = [&](int tile) -> int {
      const int tbase = t0 + tile * kTK + ld_tg * NPT;
      int page = -1;
      if (tile < ntiles && tbase < ke && tbase + NPT > kb) {
        const int j = tbase >> shift;
        if (j < npages_grp) page = pages[j];
      }
      return page;
    };
    // Global -> register staging of one tile.
    V16 kst[NPT], vst[NPT];
    uint32_t vflags = 0;
    auto gather = [&](int tile, int page) {
      const int tbase = t0 + tile * kTK + ld_tg * NPT;
      const bool page_ok = page >= 0 && page < p.num_pages;
      vflags = 0;
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int t = tbase + u;
        const bool v = page_ok && t >= kb && t < ke;
        vflags |= (v ? 1u : 0u) << (8 * u);
        const int64_t off = (((int64_t)page << shift) + (t & (P - 1))) * row_stride + hk * D * ES + ld_c * 16;
        kst[u] = load16_or_zero(kg, off, v);
        vst[u] = load16_or_zero(vg, off, v);
      }
    };
    // Registers -> LDS buffer: K and V row-major, flags.
    auto stash = [&](int buf) {
      char* ks_s = smem + buf * BUF;
      char* vs_s = ks_s + KBYTES;
      char* fl_s = vs_s + KBYTES;
#pragma unroll
      for (int u = 0; u < NPT; ++u) {
        const int off = (ld_tg * NPT + u) * STRIDE + ld_c * 16;
        *reinterpret_cast<uint4*>(ks_s + off) = make_uint4(kst[u].w[0], kst[u].w[1], kst[u].w[2], kst[u].w[3]);
        *reinterpret_cast<uint4*>(vs_s + off) = make_uint4(vst[u].w[0], vst[u].w[1], vst[u].w[2], vst[u].w[3]);
      }
      if (ld_c == 0) {
        if constexpr (NPT == 4)
          *reinterpret_cast<uint32_t*>(fl_s + ld_tg * NPT) = vflags;
        else
          *reinterpret_cast<uint16_t*>(fl_s + ld_tg * NPT) = (uint16_t)vflags;
      }
    };

    int pg_next = -1;
    if (ntiles > 0) {
      const int pg0 = page_of(0);
      pg_next = page_of(1);
      gather(0, pg0);
      stash(0);
      __syncthreads();
    }
    for (int ti = 0; ti < ntiles; ++ti) {
      const int cur = ti & 1;
      if (ti + 1 < ntiles) {
        const int pg = pg_next;
        pg_next = page_of(ti + 2);   // consumed next iteration: its latency hides behind this one
        gather(ti + 1, pg);
      }
      if (wave_active) {
        const char* ks_s = smem + cur * BUF;
        const char* vs_s = ks_s + KBYTES;
        const char* fl_s = vs_s + KBYTES;
        // S^T[mt][nt]: tokens mt*16 + 4*lg + i, query column nt*16 + l16.
        f4_t s[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          s[mt][0] = f4_t{0.f, 0.f, 0.f, 0.f};
          s[mt][1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const V16 a = lds_load16(ks_s + (mt * 16 + l16) * STRIDE + (ks * 32 + 8 * lg) * ES);
            s[mt][0] = Mfma<T>::run(a, qb[0][ks], s[mt][0]);
            s[mt][1] = Mfma<T>::run(a, qb[1][ks], s[mt][1]);
          }
        }
        uint32_t fl[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fl[mt] = *reinterpret_cast<const uint32_t*>(fl_s + mt * 16 + 4 * lg);
        // Tiles whose 64 tokens are all valid (every tile but the ragged ends) skip masking.
        const bool full = wave_all((fl[0] & fl[1] & fl[2] & fl[3]) == 0x01010101u);
        if (!full) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool v = (fl[mt] >> (8 * i)) & 1u;
              s[mt][0][i] = v ? s[mt][0][i] : kNegInf;
              s[mt][1][i] = v ? s[mt][1][i] : kNegInf;
            }
        }
        V16 pb[2][2];   // P^T operands [nt][contraction step]
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float mx = kNegInf;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][nt][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mn = fmaxf(m_run[nt], mx * p.scale_log2);
          const float mu = (mn == kNegInf) ? 0.f : mn;
          const float alpha = fast_exp2(m_run[nt] - mu);
          m_run[nt] = mn;
          float psum = 0.f;
          float pr[4][4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // P enters the PV product rounded to the operand type, but the denominator
              // (and so the LSE) sums the fp32 weights: with bf16, summing rounded weights
              // would move LSE by up to 2^-9.
              pr[mt][i] = fast_exp2(fmaf(s[mt][nt][i], p.scale_log2, -mu));
              psum += pr[mt][i];
            }
          l_run[nt] = l_run[nt] * alpha + psum;
          // Once the running maxima settle, alpha is 1 on every lane: skip the rescale.
          if (!wave_all(alpha == 1.f)) {
#pragma unroll
            for (int dm = 0; dm < DM; ++dm) oacc[dm][nt] *= alpha;
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            pb[nt][kk].w[0] = Mfma<T>::pack(pr[2 * kk][0], pr[2 * kk][1]);
            pb[nt][kk].w[1] = Mfma<T>::pack(pr[2 * kk][2], pr[2 * kk][3]);
            pb[nt][kk].w[2] = Mfma<T>::pack(pr[2 * kk + 1][0], pr[2 * kk + 1][1]);
            pb[nt][kk].w[3] = Mfma<T>::pack(pr[2 * kk + 1][2], pr[2 * kk + 1][3]);
          }
        }
        // O^T[dm][nt] += V^T * P^T.  Contraction step kk covers tokens kk*32 .. +32; lane
        // group g supplies contraction elements 8g .. 8g+7 = tokens kk*32 + 16h + 4g + i
        // (h = 0, 1; i = 0..3), the order of the S^T accumulators; each half is one
        // transpose read of rows kk*32 + 16h + 4g + tr_row, columns dm*16 + 4*tr_piece.
#pragma unroll
        for (int dm = 0; dm < DM; ++dm)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const char* base = vs_s + (kk * 32 + 4 * lg + tr_row) * STRIDE + (dm * 16 + 4 * tr_piece) * ES;
            const uint2 lo = lds_read_tr(base);
            const uint2 hi = lds_read_tr(base + 16 * STRIDE);
            V16 a;
            a.w[0] = lo.x; a.w[1] = lo.y; a.w[2] = hi.x; a.w[3] = hi.y;
            oacc[dm][0] = Mfma<T>::run(a, pb[0][kk], oacc[dm][0]);
            oacc[dm][1] = Mfma<T>::run(a, pb[1][kk], oacc[dm][1]);
          }
      }
      if (ti + 1 < ntiles) stash(cur ^ 1);
      __syncthreads();
    }

    // Finish: total sum over the 4 lane groups, normalise, write the fp32 state.
    if (wave_active) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float lt = l_run[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int r = wv * kRowsPerWave + nt * 16 + l16;
        if (r < nrows) {
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          const int64_t srow_q = (int64_t)srow + r / G;
          const int h = hk * G + r % G;
          float* dst = p.st_o + (srow_q * p.hq + h) * D;
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) {
            const f4_t o = oacc[dm][nt] * inv;
            *reinterpret_cast<float4*>(dst + dm * 16 + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
          }
          if (lg == 0)
            p.st_lse[srow_q * p.hq + h] = lt > 0.f ? (m_run[nt] + log2f(lt)) * kLn2 : kNegInf;
        }
      }
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_prefix_t(const PrefixParams& p, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, p.hkv), block(kThreads);
  hipLaunchKernelGGL((prefix_kernel<T, D, G>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_prefix_g(int group, const PrefixParams& p, int grid_x, hipStream_t s) {
  switch (group) {
    case 1: return launch_prefix_t<T, D, 1>(p, grid_x, s);
    case 2: return launch_prefix_t<T, D, 2>(p, grid_x, s);
    case 4: return launch_prefix_t<T, D, 4>(p, grid_x, s);
    case 8: return launch_prefix_t<T, D, 8>(p, grid_x, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_prefix_d(int head_dim, int group, const PrefixParams& p, int grid_x,
                                  hipStream_t s) {
  if (head_dim == 64) return launch_prefix_g<T, 64>(group, p, grid_x, s);
  if (head_dim == 128) return launch_prefix_g<T, 128>(group, p, grid_x, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefix(pkc_dtype dt, int head_dim, int group, int tile_q, const PrefixParams& p,
                         int grid_x, hipStream_t s) {
  if (grid_x <= 0) return hipSuccess;
  if (tile_q * group > 4 * kRowsPerWave) return hipErrorInvalidValue;
  switch (dt) {
    case PKC_F16: return launch_prefix_d<F16>(head_dim, group, p, grid_x, s);
    case PKC_BF16: return launch_prefix_d<BF16>(head_dim, group, p, grid_x, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
