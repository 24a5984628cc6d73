// Multi-query attention over a shared KV run (one cascade level) for gfx950, on MFMA.
//
// "Cascade Inference" blog, algorithm step 1 and Fig. 3: the queries of all requests that
// share a prefix attend to it together, so the prefix KV is staged once on chip and reused by
// every query instead of being fetched once per request.  The FlashInfer paper summary
// (section A3, composable formats) describes the same thing as a dense block of the KV
// block-sparse matrix processed with a large row tile.  Many queries against one KV set is a
// real dense contraction, so both products run on matrix cores.
//
// Tile stream = 4 waves = 128 query rows (a row is one (query, head) pair of the KV head's
// group; heads of one query are adjacent rows).  A workgroup runs one tile stream (4 waves,
// two workgroups per compute unit) or two streams over alternate tiles of its item (8 waves,
// one workgroup per compute unit), whose states are merged through LDS at the end.
//
// KV streaming: 32-token tiles go straight from HBM into a 4-stage LDS ring per stream with
// buffer loads that write LDS (no register staging), so three tiles (48 KB per stream) are in
// flight while one is computed.  Each load instruction moves 1 KB: whole 16-byte chunks of a few
// head_dim-contiguous K (or V) rows of one page, through a buffer resource over that page.
// Rows outside the item's token range and pages outside [0, num_pages) are out of the
// resource's range, so the hardware writes zeros to LDS and reads nothing.  Chunk positions
// inside a row are XOR-swizzled by the row so that the matrix-core operand reads below hit
// distinct LDS banks; the swizzle is applied on the global side (each lane fetches the chunk
// that belongs at its LDS position).
//
// Per tile and wave (32 query rows):
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16} (tokens are the M dimension, so each lane
//     owns one query column and the softmax reductions are mostly in-lane);
//   * online softmax in base 2 (running max / sum per query), masked by the tile's valid-token
//     bits (range and page validity, computed on the scalar unit);
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T accumulators, and V^T's
//     operand is read with the gfx950 LDS transpose read (ds_read_b64_tr_b16), which hands
//     each lane one head_dim column of four consecutive token rows.
// Output: one fp32 state (O normalised, natural-log LSE) per (query, head, item).
//
// FP8 pools (F8, OCP E4M3 codes with 16-bit queries; FlashInfer paper summary, appendix F):
// the ring holds the codes (half the bytes per tile, so twice the tiles in flight), and the
// codes are converted in registers on their way from LDS into the matrix-core operands: 8
// bytes per lane per operand (ds_read_b64 for K, the 8-bit transpose read for V^T), 4
// packed conversions each.  Every E4M3 value is exact in fp16 and bf16, so the arithmetic
// is that of the 16-bit path; the pool scales act outside the loop (K's on the softmax scale,
// V's on the final state).
//
// This header holds the kernel template; prefix.hip instantiates the 16-bit pools and
// prefix_fp8.hip the FP8 ones.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkc {

namespace prefix_detail {

constexpr int kTK = 32;        // KV tokens per tile
constexpr int kWavesPerStream = 4;  // 4 waves x 32 query rows = one 128-row tile
constexpr int kRowsPerWave = 32;
constexpr float kSlack = 8.f;  // lazy-rescale margin of the running maximum, log2 units

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

// True on every lane when `pred` holds on some active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lane groups that hold one
// query column of an S^T tile), with the gfx950 lane-swap instructions: permlane32_swap of a
// value with itself leaves lanes l and l ^ 32 in the two results, permlane16_swap likewise
// for l ^ 16.
__device__ __forceinline__ float lane_groups_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_groups_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

// Buffer resource words for the LDS-writing loads below (raw addressing, no swizzle, the
// same word 3 as make_rsrc): `bytes` bytes at `base`; an offset at or past `bytes` reads zeros.
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u4_t dma_rsrc(const void* base, int32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes, (uint32_t)kBufferWord3};
}

// Nontemporal buffer load of 16 bytes per lane straight into LDS: lane l writes lds + 16 * l
// (M0 holds the LDS address).  Written as an asm statement, so the compiler neither moves
// memory accesses across it nor adds waits of its own for it: the ring below orders these
// loads against the LDS reads with explicit vector-memory waits and barriers.
// m0 is the LDS byte address.  The descriptor and the scalar offset are wave-uniform by
// construction; readfirstlane states that to the compiler (a no-op on scalar registers).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void load_lds16(u4_t r, uint32_t m0, int32_t voff, int32_t soff) {
  u4_t rs;
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)r[i]);
  const int32_t ss = __builtin_amdgcn_readfirstlane(soff);
  __asm__ volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rs), "s"(ss), "{m0}"(m0)
                   : "memory");
}

// 16-byte global load whose completion the caller orders with an explicit vector-memory wait
// (the compiler does not count the asm loads above, so it must not place that wait itself).
// The value must pass through ready() after the wait and before its first use.
__device__ __forceinline__ u4_t load16_async(const void* p) {
  u4_t x;
  __asm__ volatile("global_load_dwordx4 %0, %1, off" : "=v"(x) : "v"(p) : "memory");
  return x;
}
__device__ __forceinline__ void ready(u4_t& x) { __asm__ volatile("" : "+v"(x)); }

// s_waitcnt on the vector-memory count only (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; the others at their maxima).
#define PKC_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)
// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima).
#define PKC_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Workgroup barrier that the compiler may not move memory accesses across (the builtin alone
// is not a memory operation); the ring's waits are explicit.
__device__ __forceinline__ void ring_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Physical 16-byte chunk of logical chunk c in LDS row r: c ^ swz(r).  D = 128 (16 chunks per
// 256-byte row): the 16 rows read by one K operand load and the 8 rows x 2 chunks of one
// transpose read land on distinct banks.  D = 64 (8 chunks per 128-byte row, two rows per bank
// sweep): the same property with the row parity selecting the bank half.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 2 * (r & 7) + ((r >> 3) & 1);
  else return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

// Physical 16-byte chunk of logical chunk c in LDS code row r (FP8 rings, D bytes per row):
// c ^ swz8(r).  D = 128 (two rows per 256-byte bank sweep): the 16 rows of one K operand read
// (8 bytes each, same column) and the 8 rows x 2 halves of one 8-bit transpose read (tokens
// 4g + i and 16 + 4g + i) land on distinct banks in each half-wave.  D = 64 (four rows per
// sweep): the same with the row's position in the sweep.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  if constexpr (D == 128) return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 2);
  else return ((r >> 2) & 3) ^ (((r >> 4) & 1) << 1);
}

// Converts 8 E4M3 codes (bytes in address order) to 8 values of the operand type T.
template <typename T>
__device__ __forceinline__ V16 e4m3x8_to_operand(uint2 c) {
  V16 r;
  const uint32_t w[2] = {c.x, c.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (std::is_same<T, F16>::value) {
      r.w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
      r.w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
    } else {
      r.w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
      r.w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
  }
  return r;
}

__device__ __forceinline__ uint2 lds_load8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

// Keeps N (4 or 8) 8-byte LDS reads together: an empty statement that takes all of their
// values makes the compiler issue every read before it waits for the first, where it would
// otherwise wait for each read right before converting it.
typedef uint32_t u2v_t __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void hold_reads(u2v_t (&x)[N]) {
  static_assert(N == 4 || N == 8, "read batch");
  if constexpr (N == 4)
    __asm__ volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  else
    __asm__ volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
}

// 8-bit transpose read: within each 16-lane group, the 8-byte pieces named by lanes 2i and
// 2i+1 form row i (16 bytes); lane j receives byte j of rows 0..7.
typedef int i2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_read_tr8(const char* p) {
  const i2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i2_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Runs f(integral_constant<S>, j + S) for S = S0 .. N-1 while j + S < n; false once it stops
// early.  Ring stages are template constants inside f, so their LDS addresses are immediates.
template <int S0, int N, typename F>
__device__ __forceinline__ bool unrolled_steps(F& f, int j, int n) {
  if constexpr (S0 < N) {
    if (j + S0 >= n) return false;
    f(std::integral_constant<int, S0>(), j + S0);
    return unrolled_steps<S0 + 1, N>(f, j, n);
  }
  return true;
}

}  // namespace prefix_detail

// F8: the K / V pools hold OCP E4M3 codes (T is the query and operand type).  CAUSAL: ragged
// multi-token queries with the causal mask (each group's queries are its last tokens).
template <typename T, int D, int G, int NS, bool F8, bool CAUSAL = false>
__global__ __launch_bounds__(64 * prefix_detail::kWavesPerStream * NS, NS == 1 ? 2 : 1) void prefix_kernel(const PrefixParams p) {
  using namespace prefix_detail;
  constexpr int ES = 2;
  constexpr int RB = D * ES;                 // bytes per 16-bit K / V row (operand tiles)
  constexpr int KB = F8 ? 1 : 2;             // pool bytes per element
  constexpr int RBG = D * KB;                // bytes per K / V row in the pool and the ring
  constexpr int CPRG = RBG / 16;             // 16-byte chunks per ring row
  constexpr int NDMA = 4;                    // load instructions per wave per tile (K and V)
  constexpr int STBG = kTK * RBG;            // bytes of K (or V) of one ring tile
  constexpr int SLOT = 2 * STBG;             // one tile in the ring: K rows, then V rows
  // Ring depth and tiles in flight: a stage is read by the arithmetic of its step, so it is
  // refilled one step later (STAGES - 1 tiles in flight: 48 KB per stream with 16-bit pools,
  // 56 KB with FP8 codes, whose half-size tiles leave room for 8 stages).
  constexpr int STAGES = F8 ? 8 : 4;
  constexpr int AHEAD = STAGES - 1;
  constexpr int KS = D / 32;                 // contraction steps of S^T
  constexpr int DM = D / 16;                 // 16-row tiles of O^T
  constexpr int RING = STAGES * NS * SLOT;
  constexpr int CBUF = 0;
  static_assert(kTK == 32 && (D == 64 || D == 128) && (NS == 1 || NS == 2), "tile layout");

  // The ring: stage s of stream g is ring + (g * STAGES + s) * SLOT; the valid-row bits of that
  // tile are word g * STAGES + s of sflag (byte w written by the stream's wave w).
  __shared__ __attribute__((aligned(16))) char smem[RING + CBUF];
  __shared__ uint32_t sflag[STAGES * NS];
  char* const ring = smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wv / kWavesPerStream;   // tiles stream, stream + NS, stream + 2 NS, ...
  const int wq = wv % kWavesPerStream;       // query rows 32 wq .., tile rows 8 wq ..
  const int l16 = lane & 15;
  const int lg = lane >> 4;              // lane group 0..3
  const int hk = blockIdx.y;
  const int shift = p.page_shift;
  const int P = p.page_size;
  const char* kg = static_cast<const char*>(p.k);
  const char* vg = static_cast<const char*>(p.v);
  const int32_t row_stride = p.hkv * RBG;       // bytes between consecutive slots of a page
  const int32_t page_bytes = P * row_stride;    // < 2 GiB (checked on the host)
  const int32_t npool = (int32_t)min<int64_t>(p.num_pages, INT32_MAX);
  // Transpose-read role inside the lane group: row (4 tokens apart) and 8-byte column piece.
  const int tr_row = (lane & 15) >> 2;
  const int tr_piece = lane & 3;

  // Loader role.  Wave wq of a stream loads tile rows 8wq .. 8wq+7 of K and of V as two 4-row
  // groups (rows 8wq + 4g .., one page each since pages hold a multiple of 4 slots).  256-byte
  // rows: one 1 KB instruction per group, lane l -> row 8wq + 4g + l/16, LDS chunk l%16.
  // 128-byte rows: one 1 KB instruction covers both groups as two exec-masked halves, lane l ->
  // row 8wq + l/8, LDS chunk l%8.  64-byte rows (FP8 codes, D = 64): lanes 0..31 cover both
  // groups the same way (lane l -> row 8wq + l/4) and lanes 32..63 load nothing.  16-bit rows
  // are swizzled (each lane fetches logical chunk (LDS chunk) ^ swz(row)); code rows likewise
  // with swz8.  voff is a lane's byte offset from its group's first row in the page.  Pages of
  // 8 or more slots hold all 8 rows of the wave: then one buffer resource pair serves both
  // groups.  Every path issues the same NDMA loads per tile (the ring's waits count them).
  constexpr int NI = RBG == 256 ? 2 : 1;   // instructions per operand per tile
  constexpr int LROWS = 64 / CPRG;         // rows one instruction covers (all lanes)
  int32_t voff[NI];
  int lrow[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = 8 * wq + (RBG == 256 ? 4 * i + lane / 16 : (lane / CPRG) % 8);
    const int cg = F8 ? (lane % CPRG) ^ swz8<D>(lrow[i]) : (lane % CPRG) ^ swz<D>(lrow[i]);
    voff[i] = ((lrow[i] - 8 * wq) & 3) * row_stride + hk * RBG + cg * 16;
  }
  const bool one_page = P >= 8;
  static_assert(LROWS >= 4, "row geometry");

  // A deferred plan: the workgroups take their own items from the host copy and copy the
  // plan's words into the workspace, thread t of the grid word t (further words, for plans
  // larger than the grid, after the items).  The copy load is issued first and
  // unconditionally (from a valid address in every case: a branch around it would make the
  // compiler wait for it), so its latency passes while the item reads below go to the host
  // buffer too; its store follows the items, once the ring has drained.  The load is older
  // than every load of the ring, so it can only lengthen the ring's vector-memory waits.
  const bool deferred = p.plan_host != nullptr;
  const int nthreads = (int)(blockDim.x * gridDim.x * gridDim.y);
  const int cw = (int)((blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x);
  const int32_t* copy_src = deferred ? p.plan_host + min(cw, max(p.plan_words - 1, 0)) : p.indptr;
  const int32_t copy_val = *copy_src;
  const int32_t* indptr_r = deferred ? p.plan_host + (p.indptr - p.plan_dev) : p.indptr;
  const int32_t* items_r = deferred ? p.plan_host + (p.items - p.plan_dev) : p.items;
  const int it_begin = scalar_load(indptr_r + blockIdx.x);
  const int it_end = scalar_load(indptr_r + blockIdx.x + 1);
  // The record of item blockIdx.x is read together with the CTA's item range: when a level
  // has one item per CTA (a decode step's shared prefix), CTA c's item is item c, and its
  // record then needs no second round trip.  (The items array holds at least #CTA records.)
  const int32_t* rec_c = items_r + 8 * (int64_t)blockIdx.x;
  int c_grp = scalar_load(rec_c), c_q0 = scalar_load(rec_c + 1), c_nq = scalar_load(rec_c + 2);
  int c_kb = scalar_load(rec_c + 3), c_ke = scalar_load(rec_c + 4), c_srow = scalar_load(rec_c + 5);
  // Both reads complete here, together (an empty statement that takes all their values keeps
  // the compiler from moving the record's reads behind the range test).
  __asm__ volatile("" : "+s"(c_grp), "+s"(c_q0), "+s"(c_nq), "+s"(c_kb), "+s"(c_ke), "+s"(c_srow)
                   : "s"(it_begin), "s"(it_end));
  for (int it = it_begin; it < it_end; ++it) {
    int grp, q0, nq, kb, ke, srow;
    if (it == (int)blockIdx.x) {
      grp = c_grp; q0 = c_q0; nq = c_nq; kb = c_kb; ke = c_ke; srow = c_srow;
    } else {
      const int32_t* rec = items_r + 8 * (int64_t)it;
      grp = scalar_load(rec);
      q0 = scalar_load(rec + 1);
      nq = scalar_load(rec + 2);
      kb = scalar_load(rec + 3);
      ke = scalar_load(rec + 4);
      srow = scalar_load(rec + 5);
    }
    const int nrows = nq * G;
    // A group's page run [pbeg, pbeg + npages_grp) is clamped into the page list, so a
    // malformed indptr cannot make the scalar loads below read past it.
    int pbeg, npages_grp;
    if (p.page_indptr) {
      pbeg = min(max(scalar_load(p.page_indptr + grp), 0), p.num_page_indices);
      npages_grp = min(max(scalar_load(p.page_indptr + grp + 1) - pbeg, 0), p.num_page_indices - pbeg);
    } else {
      pbeg = grp * p.table_stride;
      npages_grp = p.table_stride;
    }
    const int32_t* pages = p.page_indices + pbeg;
    // Causal mask: query i of the item (rows i * G ..) sees tokens t <= lim0 + i, where lim0
    // is the limit of the item's first query (its queries are the group's last l_q tokens).
    // Tokens past the last query's limit are not visited at all.
    int lim0 = 0;
    // Tree mask of the group (causal variant): its new tokens start at tbase, the item's first
    // query is the group's query tq0, and (query qi, token t >= tbase) is byte
    // tmoff + qi * tlq + (t - tbase) of the mask.
    int tbase = 0, tq0 = 0, tlq = 0, tmoff = 0;
    if constexpr (CAUSAL) {
      const int gq0 = scalar_load(p.grp_qo_indptr + grp), gq1 = scalar_load(p.grp_qo_indptr + grp + 1);
      const int kvl = scalar_load(p.grp_kv_lens + grp);
      lim0 = kvl - (gq1 - gq0) + (q0 - gq0);
      ke = min(ke, lim0 + nq);
      if (p.tree_mask) {
        tlq = gq1 - gq0;
        tbase = kvl - tlq;
        tq0 = q0 - gq0;
        tmoff = scalar_load(p.mask_indptr + grp);
      }
    }
    const int t0 = (kb / kTK) * kTK;
    // A group without pages holds no tokens (its kv_len is then a caller error).
    const int ntiles = (ke > kb && npages_grp > 0) ? (ke - t0 + kTK - 1) / kTK : 0;
    const int nsteps = (ntiles + NS - 1) / NS;   // tiles per stream, rounded up
    const int last_page = max(npages_grp - 1, 0);
    const bool wave_active = wq * kRowsPerWave < nrows;

    // Page-list entries of this wave's two row groups in tile tt (scalar loads, clamped into
    // the list; a group past the list is rejected when the tile is issued).  They are fetched
    // one step before use, so their latency hides behind a tile's arithmetic.
    struct Pg { int e0, e1; };
    // Every lambda here is forced inline: one left out of line takes the kernel parameters by
    // reference, which moves them to scratch memory and every address computation with them to
    // the vector unit.
    auto fetch = [&](int tt) __attribute__((always_inline)) -> Pg {
      const int rb = t0 + tt * kTK + 8 * wq;
      Pg r;
      r.e0 = scalar_load(pages + min(rb >> shift, last_page));
      // One page holds all 8 rows: the second entry is not read (a copy of the first would
      // make the wave wait for its load here instead of at the next step's barrier).
      r.e1 = one_page ? 0 : scalar_load(pages + min((rb + 4) >> shift, last_page));
      return r;
    };

    // Loads of tile tt into slot `dst` and the slot's valid-row byte of this wave; a tile past
    // the end reads nothing (zeros) and marks no row valid.
    // dst is the LDS byte address of the slot.
    auto issue = [&](int tt, const Pg& pg, uint32_t dst, uint32_t* flag) __attribute__((always_inline)) {
      const int rb = t0 + tt * kTK + 8 * wq;      // token of the wave's first row
      const bool in_tiles = tt < ntiles;
      uint32_t okbits;
      if (one_page) {
        // The wave's 8 rows sit in one page: one resource pair, row offsets from its first row.
        const bool ok = in_tiles & ((rb >> shift) < npages_grp) & (pg.e0 >= 0) & (pg.e0 < npool);
        const int64_t pofs = ok ? (int64_t)pg.e0 * page_bytes : 0;
        const u4_t rk = dma_rsrc(kg + pofs, ok ? page_bytes : 0);
        const u4_t rw = dma_rsrc(vg + pofs, ok ? page_bytes : 0);
        const int32_t soff = (rb & (P - 1)) * row_stride;   // group g: + 4 g rows
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int t = t0 + tt * kTK + lrow[i];
          const int32_t off = ((t >= kb) & (t < ke)) ? voff[i] : kOffsetNone;
          const uint32_t dk = dst + (8 * wq + 4 * i) * RBG;
          const uint32_t dv = dk + STBG;
          if constexpr (RBG == 256) {
            load_lds16(rk, dk, off, soff + 4 * i * row_stride);
            load_lds16(rw, dv, off, soff + 4 * i * row_stride);
          } else {
            constexpr int HALF = 4 * CPRG;   // lanes of one 4-row group
            if (lane < HALF) {
              load_lds16(rk, dk, off, soff);
              load_lds16(rw, dv, off, soff);
            } else if (lane < 2 * HALF) {
              load_lds16(rk, dk, off, soff + 4 * row_stride);
              load_lds16(rw, dv, off, soff + 4 * row_stride);
            }
          }
        }
        okbits = ok ? 0xFFu : 0u;
      } else {
        const int e[2] = {pg.e0, pg.e1};
        u4_t rk[2], rw[2];
        int32_t soff[2];
        bool ok[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int tg = rb + 4 * g;
          ok[g] = in_tiles & ((tg >> shift) < npages_grp) & (e[g] >= 0) & (e[g] < npool);
          const int64_t pofs = ok[g] ? (int64_t)e[g] * page_bytes : 0;
          rk[g] = dma_rsrc(kg + pofs, ok[g] ? page_bytes : 0);
          rw[g] = dma_rsrc(vg + pofs, ok[g] ? page_bytes : 0);
          soff[g] = (tg & (P - 1)) * row_stride;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int t = t0 + tt * kTK + lrow[i];
          const int32_t off = ((t >= kb) & (t < ke)) ? voff[i] : kOffsetNone;
          const uint32_t dk = dst + (8 * wq + 4 * i) * RBG;
          const uint32_t dv = dk + STBG;
          if constexpr (RBG == 256) {
            load_lds16(rk[i], dk, off, soff[i]);
            load_lds16(rw[i], dv, off, soff[i]);
          } else {
            // Two exec-masked halves (their rows may sit in different pages); both write the
            // block's 8 rows, lane l at 16 * l.
            constexpr int HALF = 4 * CPRG;   // lanes of one 4-row group
            if (lane < HALF) {
              load_lds16(rk[0], dk, off, soff[0]);
              load_lds16(rw[0], dv, off, soff[0]);
            } else if (lane < 2 * HALF) {
              load_lds16(rk[1], dk, off, soff[1]);
              load_lds16(rw[1], dv, off, soff[1]);
            }
          }
        }
        okbits = (ok[0] ? 0x0Fu : 0u) | (ok[1] ? 0xF0u : 0u);
      }
      // Valid rows: inside [kb, ke) and in a valid page.
      const int lo = min(max(kb - rb, 0), 8), hi = min(max(ke - rb, 0), 8);
      uint32_t bits = hi > lo ? (((1u << hi) - 1u) & ~((1u << lo) - 1u)) : 0u;
      bits &= okbits;
      reinterpret_cast<uint8_t*>(flag)[wq] = (uint8_t)bits;
    };

    V16 qb[2][KS];   // Q^T operands: query row wq*32 + nt*16 + l16, head_dim ks*32 + 8*lg .. +8
    f4_t oacc[DM][2];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) oacc[dm][nt] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {kNegInf, kNegInf};
    float l_run[2] = {0.f, 0.f};
    // Derived from m_run, refreshed only when it moves: the raise bound m_run + kSlack and
    // the exponent offset -mu (mu = m_run, or 0 while the column has seen no score).
    float m_lim[2] = {kNegInf, kNegInf};
    float nmu[2] = {-0.f, -0.f};

    // Per lane and query tile nt: the causal limit of the lane's query column minus the offset
    // 4 * lg of its first S^T row, so that element (mt, i) of a tile starting at token tok0 is
    // masked when tok0 + 16 mt + i > cbase[nt].  Causal masking is a compile-time variant, so
    // the kernels without it carry none of its per-tile work.
    int cbase[2] = {0, 0};
    if constexpr (CAUSAL) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) cbase[nt] = lim0 + (wq * kRowsPerWave + nt * 16 + l16) / G - 4 * lg;
    }
    // Software pipeline inside each wave (kPipe): the step of tile j runs the S^T products of
    // tile j while the vector ALU finishes the softmax of tile j-1, then tile j-1's PV
    // products, then reads tile j's V^T operands into registers.  Every LDS read of a tile
    // still happens in the tile's own step, so the ring protocol is unchanged; the operands,
    // scores and weights of one tile are exactly those of the unpipelined order.  A dummy
    // previous tile (scores -inf, V^T operands zero) starts the pipeline: its weights are 0
    // and it adds nothing.  The pipeline keeps a second score tile and the V^T operands live
    // across the step (about 250 VGPRs at D = 128); with grouped heads at D = 128 the extra
    // row indexing no longer fits 256, so those instantiations run a tile's pieces in order
    // in its step.
    constexpr bool kPipe = D == 64 || G == 1;
    f4_t sp[2][2];   // scores of the previous tile, waiting for their softmax
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sp[mt][nt] = f4_t{kNegInf, kNegInf, kNegInf, kNegInf};
    uint32_t mask_p = ~0u;   // valid-token bits and first token of the previous tile
    int tok0_p = 0;
    V16 va[DM];      // V^T operands of the previous tile
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) va[dm] = zero16();

    // S^T[mt][nt] of a tile: tokens mt*16 + 4*lg + i, query column nt*16 + l16.  The K
    // operands of each 16-token half are read together, then used by that half's products.
    // FP8 code operands: codes ks*32 + 8*lg .. +8 of K row r, half lg & 1 of logical chunk
    // 2 ks + lg / 2.  With the in-wave pipeline every code read of a tile is issued before
    // the first wait (8 K reads at D = 128, then 8 V^T reads); the in-order step has no
    // registers to spare for that and converts each read as it arrives.
    auto kcode = [&](const char* ks_s, int r, int ks) __attribute__((always_inline)) {
      return lds_load8(ks_s + r * RBG + (((2 * ks + (lg >> 1)) ^ swz8<D>(r)) * 16) + (lg & 1) * 8);
    };
    auto score = [&](const char* ks_s, f4_t (&s)[2][2]) __attribute__((always_inline)) {
      if constexpr (F8 && kPipe) {
        u2v_t kc[2 * KS];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            kc[mt * KS + ks] = __builtin_bit_cast(u2v_t, kcode(ks_s, mt * 16 + l16, ks));
          }
        hold_reads(kc);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          V16 ka[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) ka[ks] = e4m3x8_to_operand<T>(__builtin_bit_cast(uint2, kc[mt * KS + ks]));
          s[mt][0] = f4_t{0.f, 0.f, 0.f, 0.f};
          s[mt][1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s[mt][0] = Mfma<T>::run(ka[ks], qb[0][ks], s[mt][0]);
            s[mt][1] = Mfma<T>::run(ka[ks], qb[1][ks], s[mt][1]);
          }
        }
        return;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = mt * 16 + l16;
        V16 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (F8)
            ka[ks] = e4m3x8_to_operand<T>(kcode(ks_s, r, ks));
          else
            ka[ks] = lds_load16(ks_s + r * RB + (((ks * 4 + lg) ^ swz<D>(r)) * 16));
        }
        s[mt][0] = f4_t{0.f, 0.f, 0.f, 0.f};
        s[mt][1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[mt][0] = Mfma<T>::run(ka[ks], qb[0][ks], s[mt][0]);
          s[mt][1] = Mfma<T>::run(ka[ks], qb[1][ks], s[mt][1]);
        }
      }
    };
    // V^T operands of a tile (see the PV products below).
    // FP8: one 8-bit transpose read per dm gives lane (l16, lg) the codes of head_dim
    // column dm*16 + l16 for its 8 tokens, in the same order: row i of the read (lanes 2i,
    // 2i+1 of the group, each naming 8 bytes of logical chunk dm) is token 4*lg + i for
    // i < 4, else 16 + 4*lg + i - 4.
    const int tr8_tok = (l16 < 8 ? 0 : 12) + 4 * lg + (l16 >> 1);
    auto vcode = [&](const char* vs_s, int dm) __attribute__((always_inline)) {
      return lds_read_tr8(vs_s + tr8_tok * RBG + ((dm ^ swz8<D>(tr8_tok)) * 16) + (l16 & 1) * 8);
    };
    auto vread = [&](const char* vs_s) __attribute__((always_inline)) {
      if constexpr (F8 && kPipe) {
        u2v_t vc[DM];
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) vc[dm] = __builtin_bit_cast(u2v_t, vcode(vs_s, dm));
        hold_reads(vc);
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) va[dm] = e4m3x8_to_operand<T>(__builtin_bit_cast(uint2, vc[dm]));
        return;
      }
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        if constexpr (F8) {
          va[dm] = e4m3x8_to_operand<T>(vcode(vs_s, dm));
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = 16 * h + 4 * lg + tr_row;
            const int c = (2 * dm + (tr_piece >> 1)) ^ swz<D>(r);
            const uint2 x = lds_read_tr(vs_s + r * RB + c * 16 + (tr_piece & 1) * 8);
            va[dm].w[2 * h] = x.x;
            va[dm].w[2 * h + 1] = x.y;
          }
        }
      }
    };
    // Softmax of the previous tile, first part: masks, each lane's share of the column
    // maxima, and the rare raise of the reference maximum (a wave-uniform branch).
    auto softmax_prepare = [&]() __attribute__((always_inline)) {
      // Tiles whose 32 tokens are all valid (every tile but the ragged ends) skip masking.
      if (mask_p != ~0u) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool v = (mask_p >> (mt * 16 + 4 * lg + i)) & 1u;
            sp[mt][0][i] = v ? sp[mt][0][i] : kNegInf;
            sp[mt][1][i] = v ? sp[mt][1][i] : kNegInf;
          }
      }
      // Causal mask, per query column.
      if constexpr (CAUSAL) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sp[mt][nt][i] = tok0_p + mt * 16 + i > cbase[nt] ? kNegInf : sp[mt][nt][i];
        // Tree mask on the tiles that reach the new tokens: a new token is visible to a query
        // where its mask byte is set (the causal limit above still applies).  Bytes of tokens
        // before the new ones are not read (an out-of-range offset reads zero).
        if (p.tree_mask != nullptr && tok0_p + kTK > tbase) {
          const rsrc_t mr = make_rsrc(p.tree_mask, p.mask_bytes);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int qi = tq0 + (wq * kRowsPerWave + nt * 16 + l16) / G;
            const int rowoff = tmoff + qi * tlq - tbase;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int t = tok0_p + mt * 16 + 4 * lg + i;
                const int32_t off = t >= tbase ? rowoff + t : kOffsetNone;
                const uint32_t vis = __builtin_amdgcn_raw_buffer_load_b8(mr, off, 0, 0);
                sp[mt][nt][i] = (t < tbase || vis != 0) ? sp[mt][nt][i] : kNegInf;
              }
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float pmx = kNegInf;   // this lane's share of the column maximum (raw scores)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) pmx = fmaxf(pmx, sp[mt][nt][i]);
        // Lazy reference maximum: m_run moves only when a score exceeds it by more than
        // kSlack (log2 units), so O and l are rescaled only on such tiles (in practice the
        // first ones).  Weights stay below 2^kSlack, which fp32 and the 16-bit operand types
        // hold with their usual relative precision, and the final state (O / l, m + log2 l)
        // does not depend on the reference used.  A fully masked column (max = -inf) never
        // raises its reference.  A column's maximum exceeds the bound exactly when one of its
        // lanes' shares does (scale_log2 > 0), so the cross-lane maximum is only formed on
        // the tiles that raise some column.
        if (wave_any(pmx * p.scale_log2 > m_lim[nt])) {
          const float mx = lane_groups_max(pmx) * p.scale_log2;
          const bool raise = mx > m_lim[nt];
          const float alpha = raise ? fast_exp2(m_run[nt] - mx) : 1.f;
          m_run[nt] = raise ? mx : m_run[nt];
          m_lim[nt] = m_run[nt] + kSlack;
          nmu[nt] = -((m_run[nt] == kNegInf) ? 0.f : m_run[nt]);
          l_run[nt] *= alpha;
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) oacc[dm][nt] *= alpha;
        }
      }
    };
    V16 pb[2];   // P^T operands per query tile nt (the tile's 32 tokens are one step)
    // bf16 weights go to the matrix cores as two bf16 terms (rounded weight and residual): a
    // single bf16 weight carries a relative error up to 2^-9, which over a few tokens with
    // values of opposite sign exceeds the output tolerance.  fp16 weights (2^-12) need not.
    constexpr bool kSplitP = std::is_same<T, BF16>::value;
    V16 pl[2];
    // Second part: the weights of the previous tile, their sums, and the operand packing.
    auto softmax_finish = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float pr[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[mt][i] = fast_exp2(fmaf(sp[mt][nt][i], p.scale_log2, nmu[nt]));
        // P enters the PV product rounded to the operand type, but the denominator (and so the
        // LSE) sums the fp32 weights: with bf16, summing rounded weights would move LSE by up
        // to 2^-9.
        float psum = pr[0][0];
#pragma unroll
        for (int k = 1; k < 8; ++k) psum += pr[k >> 2][k & 3];
        l_run[nt] += psum;
        pb[nt].w[0] = Mfma<T>::pack(pr[0][0], pr[0][1]);
        pb[nt].w[1] = Mfma<T>::pack(pr[0][2], pr[0][3]);
        pb[nt].w[2] = Mfma<T>::pack(pr[1][0], pr[1][1]);
        pb[nt].w[3] = Mfma<T>::pack(pr[1][2], pr[1][3]);
        if constexpr (kSplitP) {
          // bf16 keeps 8 bits of each weight; the residual weight - bf16(weight), rounded to
          // bf16 again, makes the product exact to about 2^-17 relative.
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t w = pb[nt].w[k];
            const float* src = pr[k >> 1] + 2 * (k & 1);
            pl[nt].w[k] = Mfma<T>::pack(src[0] - __uint_as_float(w << 16), src[1] - __uint_as_float(w & 0xffff0000u));
          }
        }
      }
    };
    // PV products of the previous tile.
    auto pv_products = [&]() __attribute__((always_inline)) {
      // O^T[dm][nt] += V^T * P^T over the tile's 32 tokens.  Lane group g supplies contraction
      // elements 8g .. 8g+7 = tokens 16h + 4g + i (h = 0, 1; i = 0..3), the order of the S^T
      // accumulators; each half is one transpose read of rows 16h + 4g + tr_row, elements
      // dm*16 + 4*tr_piece .. +4 (logical chunk 2*dm + tr_piece/2, swizzled by row).
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const V16& a = va[dm];
        oacc[dm][0] = Mfma<T>::run(a, pb[0], oacc[dm][0]);
        oacc[dm][1] = Mfma<T>::run(a, pb[1], oacc[dm][1]);
        if constexpr (kSplitP) {
          oacc[dm][0] = Mfma<T>::run(a, pl[0], oacc[dm][0]);
          oacc[dm][1] = Mfma<T>::run(a, pl[1], oacc[dm][1]);
        }
      }
    };
    auto compute = [&](const char* ks_s, const char* vs_s, uint32_t mask, int tok0) __attribute__((always_inline)) {
      if (!wave_active) return;
      if constexpr (kPipe) {
        softmax_prepare();
        f4_t s[2][2];
        score(ks_s, s);
        softmax_finish();
        pv_products();
        vread(vs_s);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) sp[mt][nt] = s[mt][nt];
        mask_p = mask;
        tok0_p = tok0;
      } else {
        score(ks_s, sp);
        mask_p = mask;
        tok0_p = tok0;
        if constexpr (!F8) vread(vs_s);   // read now: the softmax below hides their latency
        softmax_prepare();
        softmax_finish();
        if constexpr (F8) vread(vs_s);
        pv_products();
      }
    };

    if (ntiles > 0) {
      // Q^T operands first (rows past the tile read the tile's first row: their columns are
      // computed but never stored).
      u4_t qr[2][KS];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int r = wq * kRowsPerWave + nt * 16 + l16;
        const int rr = r < nrows ? r : 0;
        const int64_t qoff = ((int64_t)(q0 + rr / G) * p.hq + hk * G + rr % G) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qr[nt][ks] = load16_async(static_cast<const char*>(p.q) + (qoff + ks * 32 + 8 * lg) * ES);
      }
      // The stream's j-th tile (tile stream + j NS) lives in stage j % STAGES.  Prologue: its
      // first AHEAD tiles in flight, page entries of the next one requested.
      char* const sring = ring + stream * STAGES * SLOT;
      uint32_t* const sfl = sflag + stream * STAGES;
      Pg pg = fetch(stream);
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) {
        issue(stream + j * NS, pg, lds_addr(sring) + j * SLOT, sfl + j);
        pg = fetch(stream + (j + 1) * NS);
      }
      // The Q loads precede the prologue's AHEAD * NDMA loads.
      PKC_WAIT_VMCNT(AHEAD * NDMA);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ready(qr[nt][ks]);
          qb[nt][ks] = V16{{qr[nt][ks][0], qr[nt][ks][1], qr[nt][ks][2], qr[nt][ks][3]}};
        }

      // Step j in stage S = j % STAGES: wait for this wave's loads of the stream's j-th tile
      // (its next AHEAD - 1 tiles stay in flight), barrier (every wave's loads and valid-row
      // byte of the step's tiles have landed and every wave is done with step j-1), refill
      // stage S-1 with the stream's tile j + AHEAD, compute tile j (its S^T products and V^T
      // reads, and tile j-1's softmax and PV products), request the page entries of tile
      // j + AHEAD + 1 (after the step's LDS reads: scalar loads and LDS reads share one counter, so an
      // LDS wait also waits for any scalar load in flight).  Before the barrier the wave waits
      // for its own LDS operations (the V^T reads at the end of the previous step), so no wave
      // still reads the stage the refill overwrites.  Every stream runs the same number of
      // steps (and barriers).  Stage numbers are compile-time constants (STAGES steps per loop
      // trip), so ring addresses are immediate offsets.

      auto step = [&](auto stage_c, int j) __attribute__((always_inline)) {
        constexpr int S = decltype(stage_c)::value;
        constexpr int N = (S + AHEAD) % STAGES;
        const int tt = stream + j * NS;
        PKC_WAIT_VMCNT((AHEAD - 1) * NDMA);
        PKC_WAIT_LGKMCNT0();
        ring_barrier();
        const uint32_t mask = sfl[S];   // the same on every lane
        issue(tt + AHEAD * NS, pg, lds_addr(sring) + N * SLOT, sfl + N);
        if (tt < ntiles) {
          const int tok0 = t0 + tt * kTK;   // the tile's first token (causal mask)
          compute(sring + S * SLOT, sring + S * SLOT + STBG, mask, tok0);
        }
        pg = fetch(tt + (AHEAD + 1) * NS);
      };
      for (int j = 0; j < nsteps; j += STAGES)
        if (!unrolled_steps<0, STAGES>(step, j, nsteps)) break;
      // Drain the pipeline: the softmax and PV products of the stream's last tile.
      if (kPipe && wave_active) {
        softmax_prepare();
        softmax_finish();
        pv_products();
      }
    }

    // Every load of the ring (including the empty ones past the last tile, which still write
    // zeros to their slot) has landed and every wave is done with the ring.
    __builtin_amdgcn_s_waitcnt(0);
    ring_barrier();

    if constexpr (NS == 2) {
      // Stream 1 hands its state to stream 0 through the idle ring: value f of lane l of wave
      // wq goes to float f * 256 + 64 wq + l.  Waves wq of the two streams hold the same rows
      // in the same lanes, so the merge is lane to lane.
      constexpr int NV = DM * 2 * 4 + 4;          // oacc, m_run[2], l_run[2]
      static_assert(NV * 256 * 4 <= RING + CBUF, "merge payload fits the ring");
      float* xf = reinterpret_cast<float*>(smem) + 64 * wq + lane;
      if (ntiles > 0) {
        if (stream == 1) {
#pragma unroll
          for (int dm = 0; dm < DM; ++dm)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) xf[((dm * 2 + nt) * 4 + i) * 256] = oacc[dm][nt][i];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            xf[(DM * 8 + nt) * 256] = m_run[nt];
            xf[(DM * 8 + 2 + nt) * 256] = l_run[nt];
          }
        }
        ring_barrier();
        if (stream == 0) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float m2 = xf[(DM * 8 + nt) * 256];
            const float l2 = xf[(DM * 8 + 2 + nt) * 256];
            const float mn = fmaxf(m_run[nt], m2);
            const float mu = (mn == kNegInf) ? 0.f : mn;
            const float a1 = fast_exp2(m_run[nt] - mu), a2 = fast_exp2(m2 - mu);
            m_run[nt] = mn;
            l_run[nt] = l_run[nt] * a1 + l2 * a2;
#pragma unroll
            for (int dm = 0; dm < DM; ++dm)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                oacc[dm][nt][i] = oacc[dm][nt][i] * a1 + xf[((dm * 2 + nt) * 4 + i) * 256] * a2;
          }
        }
      }
    }

    // Finish (stream 0): total sum over the 4 lane groups, normalise, write the state.
    if (stream == 0 && wave_active) {
      // The fp32 state of a row is D contiguous floats, but a lane holds 4-float pieces of it
      // (the accumulator layout), so a direct store instruction would write 16 rows x 64 bytes.
      // Instead each wave stages 16 rows at a time in its own part of the idle ring (past the
      // stream hand-off values; rows padded by 16 bytes so they start on different banks) and
      // stores whole rows: every instruction writes 64 / (D / 4) rows of D * 4 bytes.  The
      // states are written once and read once by a later kernel, so the stores are
      // nontemporal: they stream to memory instead of filling the L2 with dirty lines that all
      // workgroups would otherwise write back together at the end of the kernel.
      constexpr int SRS = D * 4 + 16;
      constexpr int HAND = NS == 2 ? (DM * 2 * 4 + 4) * 256 * 4 : 0;
      static_assert(HAND + kWavesPerStream * 16 * SRS <= RING + CBUF, "state staging fits the ring");
      char* const stage = smem + HAND + wq * 16 * SRS;
      constexpr int LPR = D / 4;      // lanes per staged row (16 bytes each)
      constexpr int RPI = 64 / LPR;   // rows per store instruction
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float lt = lane_groups_sum(l_run[nt]);
        const int r = wq * kRowsPerWave + nt * 16 + l16;
        float inv = lt > 0.f ? 1.f / lt : 0.f;
        if constexpr (F8) inv *= p.v_scale;
        const int h = hk * G + r % G;
        const float lse_r = lt > 0.f ? (m_run[nt] + log2f(lt)) * kLn2 : kNegInf;
        if (srow >= 0) {
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) {
            const f4_t o = oacc[dm][nt] * inv;
            *reinterpret_cast<float4*>(stage + l16 * SRS + (dm * 16 + 4 * lg) * 4) = make_float4(o[0], o[1], o[2], o[3]);
          }
          if (lg == 0 && r < nrows) __builtin_nontemporal_store(lse_r, p.st_lse + ((int64_t)srow + r / G) * p.hq + h);
#pragma unroll
          for (int k = 0; k < 16 / RPI; ++k) {
            const int rr = k * RPI + lane / LPR;
            const int row = wq * kRowsPerWave + nt * 16 + rr;
            const f4_t x = *reinterpret_cast<const f4_t*>(stage + rr * SRS + (lane % LPR) * 16);
            if (row < nrows) {
              const int64_t q = (int64_t)srow + row / G;
              __builtin_nontemporal_store(x, reinterpret_cast<f4_t*>(p.st_o + (q * p.hq + hk * G + row % G) * D + (lane % LPR) * 4));
            }
          }
          // The next half's staging writes stay behind this half's reads (one wave's LDS
          // operations complete in order; this keeps the compiler from reordering them).
          __asm__ volatile("" ::: "memory");
        } else if (p.o && r < nrows) {
          // Write-through: the tile is its rows' only item, so this is their final output
          // (O rounded once to the operand type).
          const int64_t orow = (int64_t)q0 + r / G;
          char* dst = static_cast<char*>(p.o) + (orow * p.hq + h) * (D * ES);
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) {
            const f4_t o = oacc[dm][nt] * inv;
            typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u2_t{Mfma<T>::pack(o[0], o[1]), Mfma<T>::pack(o[2], o[3])},
                                        reinterpret_cast<u2_t*>(dst + (dm * 16 + 4 * lg) * ES));
          }
          if (lg == 0) __builtin_nontemporal_store(lse_r, p.lse + orow * p.hq + h);
        }
      }
    }
    // The merge reads of the ring and this item's stores are done and every wave has left the
    // ring before the next item refills it.
    __builtin_amdgcn_s_waitcnt(0);
    ring_barrier();
  }
  if (deferred) {
    if (cw < p.plan_words) p.plan_dev[cw] = copy_val;
    for (int w = cw + nthreads; w < p.plan_words; w += nthreads) p.plan_dev[w] = p.plan_host[w];
  }
}

template <typename T, int D, int G, bool F8, bool CAUSAL>
inline hipError_t launch_prefix_t(int streams, const PrefixParams& p, int grid_x, hipStream_t s) {
  const dim3 grid(grid_x, p.hkv);
  constexpr int W = prefix_detail::kWavesPerStream;
  if (streams == 2)
    hipLaunchKernelGGL((prefix_kernel<T, D, G, 2, F8, CAUSAL>), grid, dim3(128 * W), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_kernel<T, D, G, 1, F8, CAUSAL>), grid, dim3(64 * W), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, bool F8, bool CAUSAL>
inline hipError_t launch_prefix_g(int group, int streams, const PrefixParams& p, int grid_x,
                                  hipStream_t s) {
  switch (group) {
    case 1: return launch_prefix_t<T, D, 1, F8, CAUSAL>(streams, p, grid_x, s);
    case 2: return launch_prefix_t<T, D, 2, F8, CAUSAL>(streams, p, grid_x, s);
    case 4: return launch_prefix_t<T, D, 4, F8, CAUSAL>(streams, p, grid_x, s);
    case 8: return launch_prefix_t<T, D, 8, F8, CAUSAL>(streams, p, grid_x, s);
  }
  return hipErrorInvalidValue;
}

// Launches the level kernel for 16-bit operand type T over 16-bit (F8 = false) or E4M3 pools,
// with the causal mask of ragged multi-token queries when CAUSAL.
template <typename T, bool F8, bool CAUSAL = false>
inline hipError_t launch_prefix_d(int head_dim, int group, int tile_q, int streams,
                                  const PrefixParams& p, int grid_x, hipStream_t s) {
  using namespace prefix_detail;
  if (grid_x <= 0) return hipSuccess;
  if (tile_q * group > kWavesPerStream * kRowsPerWave) return hipErrorInvalidValue;
  if (p.page_size < 4 || (streams != 1 && streams != 2)) return hipErrorInvalidValue;
  if (head_dim == 64) return launch_prefix_g<T, 64, F8, CAUSAL>(group, streams, p, grid_x, s);
  if (head_dim == 128) return launch_prefix_g<T, 128, F8, CAUSAL>(group, streams, p, grid_x, s);
  return hipErrorInvalidValue;
}

}  // namespace pkc
