// fa_bwd.hip -- backward pass launches: plain, causal and dropout.
//
// The kernels and their launch template are in fa_bwd_kernels.hpp. This file
// is compiled with the MFMAs in VGPR form (-mllvm -amdgpu-mfma-vgpr-form=1):
// where a wave needs more than 256 registers (the 32-key dK/dV kernel and the
// one-workgroup dQ at d = 128, which dropout uses) the compiler's default puts
// MFMA results in AGPRs, whence every S and dP value is copied back for the
// vector math. The VGPR form cuts those copies and measured faster on the
// causal GQA backward when it ran those kernels; the sliding-window
// instantiations (fa_bwd_window.hip) measured faster with the default.
#include "fa_bwd_kernels.hpp"

namespace fa {

hipError_t launch_bwd(BwdArgs a, int d, bool causal, hipStream_t stream) {
  if (a.drop.t != 0) {
    if (d == 64) return causal ? launch<64, true, false, true>(a, stream) : launch<64, false, false, true>(a, stream);
    return causal ? launch<128, true, false, true>(a, stream) : launch<128, false, false, true>(a, stream);
  }
  if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
