// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) with in-tile products and
// segment masks (F_SEG), or dropout with segment masks when given
// (F_SEG | F_DROP, extras.hpp).
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16_it_ext(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_DROP) return dispatch_qit<F_SEG | F_DROP>(flags, a, B, s);
  return dispatch_qit<F_SEG>(flags, a, B, s);
}

}  // namespace relpos
