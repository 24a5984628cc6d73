// Device helpers of the merge operator over attention states ("Attention States and Recursive
// Attention", n-ary merge equation; the maximum LSE is subtracted for stability), shared by the
// merge kernels and by the decode kernel's in-kernel contraction, so that both produce the
// same bits.  One thread owns 4 consecutive head_dim elements of one (output, head); states
// stream through in order with a running maximum kept in base 2.
#pragma once

#include "device_common.h"

namespace pkc {

template <typename T>
__device__ __forceinline__ void load4(const void* base, int64_t idx, float* out) {
  if constexpr (Elem<T>::kBytes == 4) {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    out[0] = Elem<T>::lo(x.x); out[1] = Elem<T>::hi(x.x);
    out[2] = Elem<T>::lo(x.y); out[3] = Elem<T>::hi(x.y);
  }
}

template <typename T>
__device__ __forceinline__ void store4(void* base, int64_t idx, const float* v) {
  if constexpr (Elem<T>::kBytes == 4) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 x;
    x.x = (uint32_t)bits16<T>(v[0]) | ((uint32_t)bits16<T>(v[1]) << 16);
    x.y = (uint32_t)bits16<T>(v[2]) | ((uint32_t)bits16<T>(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = x;
  }
}

// Running merge of one more state (natural-log LSE `lse`, values o4) into (m, l, acc).
__device__ __forceinline__ void absorb(float& m, float& l, float* acc, float lse, const float* o4) {
  const float s = lse * kLog2e;
  const float mn = fmaxf(m, s);
  const float mu = (mn == kNegInf) ? 0.f : mn;
  const float a = fast_exp2(m - mu);
  const float w = fast_exp2(s - mu);
  l = l * a + w;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = acc[e] * a + o4[e] * w;
  m = mn;
}

// Normalised values and natural-log LSE of a merged state; the identity (0, -inf) when
// nothing was merged.
__device__ __forceinline__ void finish(float m, float l, float* acc, float* lse_out) {
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = l > 0.f ? acc[e] * inv : 0.f;
  *lse_out = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
}

// Loads of one fp32 state piece (4 values and the LSE).  COHERENT: device-scope atomic loads,
// which see states that other workgroups of the running kernel wrote with device-scope atomic
// stores (no cache flush or invalidation needed); otherwise plain loads (states of earlier
// kernels).
template <bool COHERENT>
__device__ __forceinline__ void load_state4(const float* st_o, const float* st_lse, int64_t oi, int64_t li,
                                            float* o4, float* ls) {
  if constexpr (COHERENT) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = __hip_atomic_load(st_o + oi + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *ls = __hip_atomic_load(st_lse + li, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    load4<F32>(st_o, oi, o4);
    *ls = st_lse[li];
  }
}

// Output (b, h), elements d0 .. d0+3: the merge of the fp32 states in rows
// merge_rows[beg .. end) of st_o / st_lse ([rows, hq, D] and [rows, hq]), written as TO.
template <typename TO, int D, bool COHERENT = false>
__device__ __forceinline__ void merge_rows_to_output(const float* st_o, const float* st_lse,
                                                     const int32_t* merge_rows, int beg, int end,
                                                     int hq, int b, int h, int d0, void* o,
                                                     float* lse) {
  float m = kNegInf, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  // Four rows' loads go out together, then are absorbed in row order (the order, and so the
  // result, is that of a one-row-at-a-time loop; only the load latency is shared).
  int k = beg;
  for (; k + 4 <= end; k += 4) {
    float o4[4][4], ls[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t r = merge_rows[k + u];
      load_state4<COHERENT>(st_o, st_lse, (r * hq + h) * D + d0, r * hq + h, o4[u], &ls[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) absorb(m, l, acc, ls[u], o4[u]);
  }
  for (; k < end; ++k) {
    const int64_t r = merge_rows[k];
    float o4[4], ls;
    load_state4<COHERENT>(st_o, st_lse, (r * hq + h) * D + d0, r * hq + h, o4, &ls);
    absorb(m, l, acc, ls, o4);
  }
  float ls;
  finish(m, l, acc, &ls);
  store4<TO>(o, ((int64_t)b * hq + h) * D + d0, acc);
  if (d0 == 0) lse[(int64_t)b * hq + h] = ls;
}

}  // namespace pkc
