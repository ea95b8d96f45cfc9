// Instantiation of the bf16 key-parallel pass (bwd_k_fast.hpp) with segment masks
// (F_SEG, extras.hpp).
#include "bwd_k_fast.hpp"

namespace relpos {

hipError_t launch_bwd_k_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_kf<F_SPLIT | F_SEG>(flags, a, B, s);
  return dispatch_kf<F_SEG>(flags, a, B, s);
}

}  // namespace relpos
