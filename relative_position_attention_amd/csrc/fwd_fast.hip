// Instantiation of the bf16 forward (fwd_fast.hpp) without the segment
// mask and dropout extras; those variants are built in fwd_seg.hip and
// fwd_drop.hip, so the three compile in parallel.
#include "fwd_fast.hpp"

namespace relpos {

hipError_t launch_attn_fwd_bf16(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_IT) return launch_attn_fwd_bf16_it(flags, a, B, s);
  if (flags & F_DROP) return launch_attn_fwd_bf16_drop(flags, a, B, s);
  if (flags & F_SEG) return launch_attn_fwd_bf16_seg(flags, a, B, s);
  if (flags & F_SPLIT) return dispatch_fast<F_SPLIT>(flags, a, B, s);
  return dispatch_fast<0>(flags, a, B, s);
}

}  // namespace relpos
