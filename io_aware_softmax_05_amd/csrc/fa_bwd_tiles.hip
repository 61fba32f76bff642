// fa_bwd_tiles.hip -- the backward pass with its second tiling (the ALT
// instantiations of the launch template in fa_bwd_kernels.hpp), behind
// fa_bwd_tiles. It exists to check that the result does not depend on the
// tile shape; its own file keeps it out of the other files' build time.
#include "fa_bwd_kernels.hpp"

namespace fa {

hipError_t launch_bwd_alt_tiles(BwdArgs a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true, false, false, true>(a, stream) : launch<64, false, false, false, true>(a, stream);
  return causal ? launch<128, true, false, false, true>(a, stream) : launch<128, false, false, false, true>(a, stream);
}

}  // namespace fa
