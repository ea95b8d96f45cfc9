// Instantiation of the bf16 key-parallel pass (bwd_k_fast.hpp) with in-tile products
// (F_IT, intile.hpp); with segment masks or dropout see bwd_k_it_ext.hip.
#include "bwd_k_fast.hpp"

namespace relpos {

hipError_t launch_bwd_k_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & (F_SEG | F_DROP)) return launch_bwd_k_bf16_it_ext(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_kit<F_SPLIT>(flags, a, B, s);
  return dispatch_kit<0>(flags, a, B, s);
}

}  // namespace relpos
