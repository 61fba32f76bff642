// fa_bwd_window.hip -- backward pass launches for the causal sliding window.
//
// The kernels and their launch template are in fa_bwd_kernels.hpp; this file
// is compiled with the compiler's default MFMA register form. It measured
// faster than the VGPR form fa_bwd.hip uses while the window ran the 32-key
// dK/dV kernel; its kernels now stay within 256 registers, where the two
// forms time the same.
#include "fa_bwd_kernels.hpp"

namespace fa {

hipError_t launch_bwd_window(BwdArgs a, int d, hipStream_t stream) {
  return d == 64 ? launch<64, true, true>(a, stream) : launch<128, true, true>(a, stream);
}

}  // namespace fa
