// Instantiation of the bf16 forward (fwd_fast.hpp) with segment masks
// (F_SEG, extras.hpp).
#include "fwd_fast.hpp"

namespace relpos {

hipError_t launch_attn_fwd_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_fast<F_SPLIT | F_SEG>(flags, a, B, s);
  return dispatch_fast<F_SEG>(flags, a, B, s);
}

}  // namespace relpos
