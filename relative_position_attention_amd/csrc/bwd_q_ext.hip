// Instantiation of the bf16 query-parallel pass (bwd_q_fast.hpp) with segment masks and
// dropout (F_EXT, extras.hpp).
#include "bwd_q_fast.hpp"

namespace relpos {

hipError_t launch_bwd_q_bf16_ext(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_SPLIT) return dispatch_qf<F_SPLIT | F_EXT>(flags, a, B, s);
  return dispatch_qf<F_EXT>(flags, a, B, s);
}

}  // namespace relpos
