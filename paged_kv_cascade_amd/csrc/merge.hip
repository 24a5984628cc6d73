// Merge kernels: n-ary merge operator over attention states ("Attention States and Recursive
// Attention", n-ary merge equation; the maximum LSE is subtracted for stability) and the
// binary merge in place.  One thread owns 4 consecutive head_dim elements of one (output,
// head); states stream through in order with a running maximum, so any number of states is
// merged in one pass.  The identity (0, -inf) results when there is nothing to merge.
#include "device_common.h"
#include "kernels.h"
#include "merge_ops.h"

namespace pkc {

// Workgroup (x, y) finishes kMergeRequestsPerBlock consecutive requests for heads
// y * HPB .. y * HPB + HPB - 1; a request the decode kernel already wrote costs one uniform
// branch.
constexpr int kMergeRequestsPerBlock = 2;
template <typename TO, int D>
__global__ __launch_bounds__(256) void merge_plan_kernel(const MergePlanParams p) {
  constexpr int TPH = D / 4;          // threads per head
  constexpr int HPB = 256 / TPH;      // heads of the block
  const int d0 = (threadIdx.x % TPH) * 4;
  const int h = blockIdx.y * HPB + threadIdx.x / TPH;
  if (h >= p.hq) return;
  for (int bi = 0; bi < kMergeRequestsPerBlock; ++bi) {
    const int b = blockIdx.x * kMergeRequestsPerBlock + bi;
    if (b >= p.batch) break;
    if (p.req_flags && p.req_flags[b]) continue;
    const int beg = p.merge_ptr[(int64_t)b * p.nl2 + p.l0];
    const int end = p.merge_ptr[(int64_t)b * p.nl2 + p.l1];
    merge_rows_to_output<TO, D>(p.st_o, p.st_lse, p.merge_rows, beg, end, p.hq, b, h, d0, p.o, p.lse);
  }
}

template <typename TI, typename TO, int D>
__global__ __launch_bounds__(256) void merge_generic_kernel(const MergeGenericParams p) {
  constexpr int TPH = D / 4;
  constexpr int HPB = 256 / TPH;
  const int i = blockIdx.x;
  const int h = blockIdx.y * HPB + threadIdx.x / TPH;
  if (h >= p.num_heads) return;
  const int d0 = (threadIdx.x % TPH) * 4;
  int beg, end;
  if (p.indptr) {
    beg = p.indptr[i];
    end = p.indptr[i + 1];
  } else {
    beg = i * p.states_per_output;
    end = beg + p.states_per_output;
  }
  float m = kNegInf, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = beg; k < end; ++k) {
    const int64_t s = p.indices ? (int64_t)p.indices[k] : (int64_t)k;
    if (s < 0 || s >= p.num_states) continue;
    float o4[4];
    load4<TI>(p.o_states, (s * p.num_heads + h) * D + d0, o4);
    absorb(m, l, acc, p.lse_states[s * p.num_heads + h], o4);
  }
  float lse;
  finish(m, l, acc, &lse);
  store4<TO>(p.o_out, ((int64_t)i * p.num_heads + h) * D + d0, acc);
  if (d0 == 0) p.lse_out[(int64_t)i * p.num_heads + h] = lse;
}

// Binary merge in place; written symmetrically in its two operands.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_inplace_kernel(void* o_a, float* lse_a,
                                                            const void* o_b,
                                                            const float* lse_b, int64_t n) {
  constexpr int TPH = D / 4;
  const int64_t sidx = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPH;
  if (sidx >= n) return;
  const int d0 = (threadIdx.x % TPH) * 4;
  float a4[4], b4[4];
  load4<T>(o_a, sidx * D + d0, a4);
  load4<T>(o_b, sidx * D + d0, b4);
  const float sa = lse_a[sidx] * kLog2e, sb = lse_b[sidx] * kLog2e;
  const float mn = fmaxf(sa, sb);
  const float mu = (mn == kNegInf) ? 0.f : mn;
  const float wa = fast_exp2(sa - mu), wb = fast_exp2(sb - mu);
  const float den = wa + wb;
  // Separately rounded products (contraction into a fused multiply-add is switched off) keep
  // the result bit-identical when a and b are swapped.
  float out[4];
  {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = a4[e] * wa;
      const float y = b4[e] * wb;
      out[e] = den > 0.f ? (x + y) / den : 0.f;
    }
  }
  // All lanes of one state sit in one wave and read lse_a in the same load instruction;
  // the store below depends on that load, so no lane can overwrite it early.
  store4<T>(o_a, sidx * D + d0, out);
  if (d0 == 0) lse_a[sidx] = den > 0.f ? (mu + log2f(den)) * kLn2 : kNegInf;
}

// Plan upload: the GPU reads the pinned host buffer directly and writes the workspace.  Being a
// kernel on the caller's queue, it needs no synchronisation with a copy engine.
__global__ __launch_bounds__(256) void plan_upload_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

hipError_t launch_plan_upload(const void* host_src, void* dev_dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = (bytes + 15) / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_upload_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(host_src), static_cast<uint4*>(dev_dst), n16);
  return hipGetLastError();
}

// Read-stream probe (measurement only): workgroup g reads bytes [g MiB, (g+1) MiB) of src,
// wave w its w-th quarter, each lane 16 bytes per load with 16 loads in flight and the
// nontemporal hint of the KV streams; one XOR per thread goes to sink so nothing is elided.
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ src,
                                                          uint32_t* __restrict__ sink) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  constexpr int kWaveBytes = 256 * 1024;
  constexpr int kLoads = kWaveBytes / 1024;     // 1 KB per wave load instruction
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const u4v* p = reinterpret_cast<const u4v*>(src) + ((int64_t)blockIdx.x * 4 + wv) * (kWaveBytes / 16) + lane;
  uint32_t acc = 0;
  for (int i = 0; i < kLoads; i += 16) {
    u4v v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = __builtin_nontemporal_load(p + (i + u) * 64);
#pragma unroll
    for (int u = 0; u < 16; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_read_stream(const void* src, int64_t mib, uint32_t* sink, hipStream_t s) {
  if (mib <= 0) return hipSuccess;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)mib), dim3(256), 0, s,
                     static_cast<const uint4*>(src), sink);
  return hipGetLastError();
}

template <typename TO>
static hipError_t merge_plan_d(int head_dim, const MergePlanParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
  const int gx = (p.batch + kMergeRequestsPerBlock - 1) / kMergeRequestsPerBlock;
  if (head_dim == 64) {
    hipLaunchKernelGGL((merge_plan_kernel<TO, 64>), dim3(gx, (p.hq + 15) / 16), dim3(256), 0, s, p);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL((merge_plan_kernel<TO, 128>), dim3(gx, (p.hq + 7) / 8), dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge_plan(pkc_dtype out_dt, int head_dim, const MergePlanParams& p,
                             hipStream_t s) {
  switch (out_dt) {
    case PKC_F32: return merge_plan_d<F32>(head_dim, p, s);
    case PKC_F16: return merge_plan_d<F16>(head_dim, p, s);
    case PKC_BF16: return merge_plan_d<BF16>(head_dim, p, s);
  }
  return hipErrorInvalidValue;
}

template <typename TI, typename TO>
static hipError_t merge_generic_d(int head_dim, const MergeGenericParams& p, hipStream_t s) {
  if (p.num_outputs <= 0) return hipSuccess;
  if (head_dim == 64) {
    dim3 grid(p.num_outputs, (p.num_heads + 15) / 16);
    hipLaunchKernelGGL((merge_generic_kernel<TI, TO, 64>), grid, dim3(256), 0, s, p);
  } else if (head_dim == 128) {
    dim3 grid(p.num_outputs, (p.num_heads + 7) / 8);
    hipLaunchKernelGGL((merge_generic_kernel<TI, TO, 128>), grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TI>
static hipError_t merge_generic_o(pkc_dtype out_dt, int head_dim, const MergeGenericParams& p,
                                  hipStream_t s) {
  switch (out_dt) {
    case PKC_F32: return merge_generic_d<TI, F32>(head_dim, p, s);
    case PKC_F16: return merge_generic_d<TI, F16>(head_dim, p, s);
    case PKC_BF16: return merge_generic_d<TI, BF16>(head_dim, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge_generic(pkc_dtype in_dt, pkc_dtype out_dt, int head_dim,
                                const MergeGenericParams& p, hipStream_t s) {
  switch (in_dt) {
    case PKC_F32: return merge_generic_o<F32>(out_dt, head_dim, p, s);
    case PKC_F16: return merge_generic_o<F16>(out_dt, head_dim, p, s);
    case PKC_BF16: return merge_generic_o<BF16>(out_dt, head_dim, p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t merge_inplace_d(int head_dim, void* o_a, float* lse_a, const void* o_b,
                                  const float* lse_b, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = n * (head_dim / 4);
  dim3 grid((unsigned)((threads + 255) / 256));
  if (head_dim == 64)
    hipLaunchKernelGGL((merge_inplace_kernel<T, 64>), grid, dim3(256), 0, s, o_a, lse_a, o_b, lse_b, n);
  else if (head_dim == 128)
    hipLaunchKernelGGL((merge_inplace_kernel<T, 128>), grid, dim3(256), 0, s, o_a, lse_a, o_b, lse_b, n);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge_inplace(pkc_dtype dt, int head_dim, void* o_a, float* lse_a,
                                const void* o_b, const float* lse_b, int64_t num_states,
                                hipStream_t s) {
  switch (dt) {
    case PKC_F32: return merge_inplace_d<F32>(head_dim, o_a, lse_a, o_b, lse_b, num_states, s);
    case PKC_F16: return merge_inplace_d<F16>(head_dim, o_a, lse_a, o_b, lse_b, num_states, s);
    case PKC_BF16: return merge_inplace_d<BF16>(head_dim, o_a, lse_a, o_b, lse_b, num_states, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
