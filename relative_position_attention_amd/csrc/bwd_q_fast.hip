// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) without the segment
// mask and dropout extras; those variants are built in bwd_q_ext.hip
// so the two halves compile in parallel.
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_EXT) return launch_bwd_q_bf16_ext(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_qf<F_SPLIT>(flags, a, B, s);
  return dispatch_qf<0>(flags, a, B, s);
}

}  // namespace relpos
