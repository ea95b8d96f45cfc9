// Instantiation of the bf16 forward (fwd_fast.hpp) without the segment
// mask and dropout extras; those variants are built in fwd_ext.hip
// so the two halves compile in parallel.
#include "fwd_fast.hpp"

namespace relpos {

hipError_t launch_attn_fwd_bf16(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_EXT) return launch_attn_fwd_bf16_ext(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_fast<F_SPLIT>(flags, a, B, s);
  return dispatch_fast<0>(flags, a, B, s);
}

}  // namespace relpos
