// Forward kernels for the wide heads (d_qk 256 with d_v 256 or 512); see
// fwd_kernel.h.  Kept in their own translation unit: these accumulators do
// not fit the VGPR file, so they keep the default AGPR allocation.
#include "fwd_kernel.h"

namespace attn {

hipError_t launch_fwd_wide(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 256 && dv == 256) return launch_cfg<256, 256, 16, 32, 2>(p, st);
  if (dqk == 256 && dv == 512) return launch_cfg<256, 512, 16, 32, 2>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
