// Instantiations of the multi-query level kernel (prefix_kernel.h) with the causal mask over
// OCP FP8 E4M3 pools (fp16 / bf16 queries), for ragged multi-token queries.
#include "prefix_kernel.h"

namespace pkc {

hipError_t launch_prefill_causal_fp8(pkc_dtype q_dt, int head_dim, int group, int tile_q, int streams,
                                     const PrefixParams& p, int grid_x, hipStream_t s) {
  switch (q_dt) {
    case PKC_F16: return launch_prefix_d<F16, true, true>(head_dim, group, tile_q, streams, p, grid_x, s);
    case PKC_BF16: return launch_prefix_d<BF16, true, true>(head_dim, group, tile_q, streams, p, grid_x, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
