// Device helpers shared by the gfx950 kernels: element types, 16-byte vectors, conversions,
// wave64 reductions inside 16-lane DPP rows, and the base-2 online-softmax primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkc {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Storage tags: the kernels move raw bits and convert explicitly.
struct F32 {};
struct F16 {};
struct BF16 {};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t u16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}
// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // RNE
}

template <typename T> __device__ __forceinline__ uint16_t bits16(float x);
template <> __device__ __forceinline__ uint16_t bits16<struct F16>(float x) { return f32_to_f16_bits(x); }
template <> __device__ __forceinline__ uint16_t bits16<struct BF16>(float x) { return f32_to_bf16_bits(x); }

template <typename T> struct Elem;
template <> struct Elem<F32> {
  static constexpr int kBytes = 4;
  __device__ static float lo(uint32_t w) { return __uint_as_float(w); }
  __device__ static void store(void* p, int64_t i, float x) { static_cast<float*>(p)[i] = x; }
};
template <> struct Elem<F16> {
  static constexpr int kBytes = 2;
  __device__ static float lo(uint32_t w) { return f16_bits_to_f32(w & 0xffffu); }
  __device__ static float hi(uint32_t w) { return f16_bits_to_f32(w >> 16); }
  __device__ static void store(void* p, int64_t i, float x) { static_cast<uint16_t*>(p)[i] = f32_to_f16_bits(x); }
};
template <> struct Elem<BF16> {
  static constexpr int kBytes = 2;
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static void store(void* p, int64_t i, float x) { static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x); }
};

// 16 bytes = one 128-bit load.
struct alignas(16) V16 {
  uint32_t w[4];
};

__device__ __forceinline__ V16 load16(const void* p) {
  V16 r;
  const uint4 x = *static_cast<const uint4*>(p);
  r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
  return r;
}
__device__ __forceinline__ V16 zero16() {
  V16 r;
  r.w[0] = r.w[1] = r.w[2] = r.w[3] = 0u;
  return r;
}

// Wave-uniform read of read-only int32 data (block tables, page lists, plan records) through
// the scalar cache.  A vector load would share the in-order vmcnt queue with the K/V stream,
// so waiting for a table entry would mean waiting for every K/V load issued before it.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

// 16 bytes at base + off when `valid`, else zeros.  The load is issued unconditionally (an
// invalid lane reads base + 0, which the caller guarantees is in bounds) and the zeros are
// selected afterwards: a branch around a load makes the compiler wait for every outstanding
// load at the branch, which would serialise a software pipeline.
__device__ __forceinline__ V16 load16_or_zero(const char* base, int64_t off, bool valid) {
  const V16 x = load16(base + (valid ? off : 0));
  V16 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r.w[k] = valid ? x.w[k] : 0u;
  return r;
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, no swizzle, 32-bit data
// format, the gfx9 word-3 encoding).  A buffer load whose offset is at or past `bytes` returns
// zeros without touching memory, so masked lanes need no select and no branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;
constexpr int32_t kOffsetNone = INT32_MIN;   // 0x80000000: past any range a kernel builds
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}
// Cache-policy operand of buffer loads: the nontemporal hint (read once, do not keep).  KV
// rows are streamed exactly once per step, and on MI355X a read stream with the hint runs
// about 10% faster than without it.
constexpr int kCachePolicyStream = 2;
template <int AUX = 0>
__device__ __forceinline__ V16 buffer_load16(rsrc_t r, int32_t off) {
  typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
  const u4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  V16 v;
  v.w[0] = x[0]; v.w[1] = x[1]; v.w[2] = x[2]; v.w[3] = x[3];
  return v;
}

// Partial dot product of the 16-byte slices of q and k (fp32 accumulate; products exact).
__device__ __forceinline__ float dot16(F32, const V16& a, const V16& b) {
  float s = __uint_as_float(a.w[0]) * __uint_as_float(b.w[0]);
  s = fmaf(__uint_as_float(a.w[1]), __uint_as_float(b.w[1]), s);
  s = fmaf(__uint_as_float(a.w[2]), __uint_as_float(b.w[2]), s);
  s = fmaf(__uint_as_float(a.w[3]), __uint_as_float(b.w[3]), s);
  return s;
}
__device__ __forceinline__ float dot16(F16, const V16& a, const V16& b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.w[i]), __builtin_bit_cast(h2_t, b.w[i]), s, false);
  return s;
}
__device__ __forceinline__ float dot16(BF16, const V16& a, const V16& b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.w[i]), __builtin_bit_cast(b2_t, b.w[i]), s, false);
  return s;
}

// Unpack a 16-byte slice to floats (VEC = 4 for f32, 8 for 16-bit types).
__device__ __forceinline__ void unpack16(F32, const V16& a, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(a.w[i]);
}
template <typename T>
__device__ __forceinline__ void unpack16(T, const V16& a, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = Elem<T>::lo(a.w[i]);
    out[2 * i + 1] = Elem<T>::hi(a.w[i]);
  }
}

// OCP FP8 E4M3 KV storage (one byte per element) with queries and outputs of the 16-bit type
// TQ.  Every E4M3 value is exact in fp16, bf16 and fp32, so the kernels convert codes with the
// gfx950 conversion instructions (scale 1) and apply the pool scales outside the inner loops:
// the K scale multiplies sm_scale, the V scale multiplies the output accumulators.
template <typename TQ> struct KV8 {};
template <typename TQ> struct Elem<KV8<TQ>> { static constexpr int kBytes = 1; };

template <typename T> struct IsKV8 { static constexpr bool value = false; };
template <typename TQ> struct IsKV8<KV8<TQ>> { static constexpr bool value = true; };
template <typename T> struct OutType { typedef T type; };
template <typename TQ> struct OutType<KV8<TQ>> { typedef TQ type; };
template <typename T> struct QBytes { static constexpr int kBytes = Elem<T>::kBytes; };
template <typename TQ> struct QBytes<KV8<TQ>> { static constexpr int kBytes = 2; };

// The q elements matching one lane's 16 bytes of K/V: 16 bytes of q for 16- and 32-bit pools,
// 32 bytes (16 fp16 / bf16 values) for FP8 pools.
template <typename T> struct QSlice { V16 v[1]; };
template <typename TQ> struct QSlice<KV8<TQ>> { V16 v[2]; };
template <typename T>
__device__ __forceinline__ QSlice<T> load_qslice(const char* qrow, int col) {
  QSlice<T> r;
  if constexpr (IsKV8<T>::value) {
    r.v[0] = load16(qrow + col * 32);
    r.v[1] = load16(qrow + col * 32 + 16);
  } else {
    r.v[0] = load16(qrow + col * 16);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ float dot16(T t, const QSlice<T>& q, const V16& k) {
  return dot16(t, q.v[0], k);
}
// Codes 4i .. 4i+3 sit in word i of the 16-byte slice (bytes in address order); the
// conversion's word select picks codes (0, 1) or (2, 3) of a word.
__device__ __forceinline__ float dot16(KV8<F16>, const QSlice<KV8<F16>>& q, const V16& k) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, false);
    const h2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, true);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.v[i >> 1].w[2 * (i & 1)]), lo, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.v[i >> 1].w[2 * (i & 1) + 1]), hi, s, false);
  }
  return s;
}
__device__ __forceinline__ float dot16(KV8<BF16>, const QSlice<KV8<BF16>>& q, const V16& k) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const b2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.w[i], 1.0f, false);
    const b2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.w[i], 1.0f, true);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.v[i >> 1].w[2 * (i & 1)]), lo, s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.v[i >> 1].w[2 * (i & 1) + 1]), hi, s, false);
  }
  return s;
}
template <typename TQ>
__device__ __forceinline__ void unpack16(KV8<TQ>, const V16& a, float* out) {
  typedef float f2v __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f2v lo = __builtin_amdgcn_cvt_pk_f32_fp8(a.w[i], false);
    const f2v hi = __builtin_amdgcn_cvt_pk_f32_fp8(a.w[i], true);
    out[4 * i] = lo[0];
    out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0];
    out[4 * i + 3] = hi[1];
  }
}

// DPP lane permutations inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// All-reduce sum over aligned groups of N lanes (N = 4, 8, 16, 32, 64).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_f<kDppQuadSwap1>(x);
  x += dpp_f<kDppQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp_f<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Base-2 attention state of one row: running max m, sum l, unnormalised accumulator.
// Merges state (m2, l2, acc2) into (m, l, acc) over n accumulator values.
template <int N>
__device__ __forceinline__ void merge_state2(float& m, float& l, float* acc, float m2, float l2,
                                             const float* acc2) {
  const float mn = fmaxf(m, m2);
  const float mu = (mn == kNegInf) ? 0.f : mn;
  const float a = fast_exp2(m - mu);
  const float b = fast_exp2(m2 - mu);
  l = l * a + l2 * b;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acc2[e] * b;
  m = mn;
}

}  // namespace pkc
