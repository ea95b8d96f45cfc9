// Instantiation of the bf16 key-parallel pass (bwd_k_fast.hpp) with in-tile products and
// segment masks (F_SEG), or dropout with segment masks when given
// (F_SEG | F_DROP, extras.hpp).
#include "bwd_k_fast.hpp"

namespace relpos {

hipError_t launch_bwd_k_bf16_it_ext(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & F_DROP) return dispatch_kit<F_SEG | F_DROP>(flags, a, B, s);
  return dispatch_kit<F_SEG>(flags, a, B, s);
}

}  // namespace relpos
