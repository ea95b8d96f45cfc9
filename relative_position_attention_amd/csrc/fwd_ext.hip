// Instantiation of the bf16 forward (fwd_fast.hpp) with segment masks and
// dropout (F_EXT, extras.hpp).
#include "fwd_fast.hpp"

namespace relpos {

hipError_t launch_attn_fwd_bf16_ext(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_fast<F_SPLIT | F_EXT>(flags, a, B, s);
  return dispatch_fast<F_EXT>(flags, a, B, s);
}

}  // namespace relpos
