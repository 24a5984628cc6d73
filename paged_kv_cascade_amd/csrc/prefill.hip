// Instantiations of the multi-query level kernel (prefix_kernel.h) with the causal mask, for
// ragged multi-token queries over fp16 / bf16 pools (the non-causal case uses the plain level
// kernel; FP8 pools are in prefill_fp8.hip).
#include "prefix_kernel.h"

namespace pkc {

hipError_t launch_prefill_causal(pkc_dtype dt, int head_dim, int group, int tile_q, int streams,
                                 const PrefixParams& p, int grid_x, hipStream_t s) {
  switch (dt) {
    case PKC_F16: return launch_prefix_d<F16, false, true>(head_dim, group, tile_q, streams, p, grid_x, s);
    case PKC_BF16: return launch_prefix_d<BF16, false, true>(head_dim, group, tile_q, streams, p, grid_x, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
