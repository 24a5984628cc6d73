// Paged batch decode over OCP FP8 E4M3 K/V pools with fp16 or bf16 queries and outputs (the
// kernel is the one in decode_kernel.h; these are its FP8 instantiations).
#include "decode_kernel.h"

namespace pkc {

hipError_t launch_decode_fp8(pkc_dtype q_dt, int head_dim, int group, int waves,
                             const DecodeParams& p, int grid_x, hipStream_t s) {
  if (grid_x <= 0) return hipSuccess;
  switch (q_dt) {
    case PKC_F16: return launch_decode_d<KV8<F16>>(head_dim, group, waves, p, grid_x, s);
    case PKC_BF16: return launch_decode_d<KV8<BF16>>(head_dim, group, waves, p, grid_x, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
