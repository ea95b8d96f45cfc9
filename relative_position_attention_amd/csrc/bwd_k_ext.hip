// Instantiation of the bf16 key-parallel pass (bwd_k_fast.hpp) with segment masks and
// dropout (F_EXT, extras.hpp).
#include "bwd_k_fast.hpp"

namespace relpos {

hipError_t launch_bwd_k_bf16_ext(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_kf<F_SPLIT | F_EXT>(flags, a, B, s);
  return dispatch_kf<F_EXT>(flags, a, B, s);
}

}  // namespace relpos
