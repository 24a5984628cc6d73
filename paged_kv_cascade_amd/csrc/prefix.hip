// Instantiations of the multi-query level kernel (prefix_kernel.h) for fp16 / bf16 pools.
#include "prefix_kernel.h"

namespace pkc {

hipError_t launch_prefix(pkc_dtype dt, int head_dim, int group, int tile_q, int streams,
                         const PrefixParams& p, int grid_x, hipStream_t s) {
  switch (dt) {
    case PKC_F16: return launch_prefix_d<F16, false>(head_dim, group, tile_q, streams, p, grid_x, s);
    case PKC_BF16: return launch_prefix_d<BF16, false>(head_dim, group, tile_q, streams, p, grid_x, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pkc
