// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) without the segment
// mask and dropout extras; those variants are built in bwd_q_seg.hip and
// bwd_q_drop.hip, so the three compile in parallel.
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_IT) return launch_bwd_q_bf16_it(flags, a, B, s);
  if (flags & F_DROP) return launch_bwd_q_bf16_drop(flags, a, B, s);
  if (flags & F_SEG) return launch_bwd_q_bf16_seg(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_qf<F_SPLIT>(flags, a, B, s);
  return dispatch_qf<0>(flags, a, B, s);
}

}  // namespace relpos
