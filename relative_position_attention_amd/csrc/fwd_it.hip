// Instantiation of the bf16 forward (fwd_fast.hpp) with in-tile products
// (F_IT, intile.hpp); with segment masks or dropout see fwd_it_ext.hip.
#include "fwd_fast.hpp"

namespace relpos {

hipError_t launch_attn_fwd_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & (F_SEG | F_DROP)) return launch_attn_fwd_bf16_it_ext(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_it<F_SPLIT>(flags, a, B, s);
  return dispatch_it<0>(flags, a, B, s);
}

}  // namespace relpos
