// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) with segment masks
// (F_SEG, extras.hpp).
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_qf<F_SPLIT | F_SEG>(flags, a, B, s);
  return dispatch_qf<F_SEG>(flags, a, B, s);
}

}  // namespace relpos
