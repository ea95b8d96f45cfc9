// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) with in-tile products
// (F_IT, intile.hpp); with segment masks or dropout see bwd_q_it_ext.hip.
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & (F_SEG | F_DROP)) return launch_bwd_q_bf16_it_ext(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_qit<F_SPLIT>(flags, a, B, s);
  return dispatch_qit<0>(flags, a, B, s);
}

}  // namespace relpos
