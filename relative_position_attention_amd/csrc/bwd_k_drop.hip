// Instantiation of the bf16 key-parallel pass (bwd_k_fast.hpp) with attention dropout
// and, when the call gives them, segment masks (F_DROP | F_SEG, extras.hpp).
#include "bwd_k_fast.hpp"

namespace relpos {

hipError_t launch_bwd_k_bf16_drop(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_kf<F_SPLIT | F_SEG | F_DROP>(flags, a, B, s);
  return dispatch_kf<F_SEG | F_DROP>(flags, a, B, s);
}

}  // namespace relpos
