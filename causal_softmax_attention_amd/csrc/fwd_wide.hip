// Forward entry for the large heads (d_qk 256 with d_v 256 or 512); the
// kernel is in fwd_large.h.  Kept in its own translation unit: its O
// accumulators keep the default AGPR allocation, which the other forward
// kernels turn off.
#include "fwd_large.h"

namespace attn {

hipError_t launch_fwd_wide(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 256 && dv == 256) return launch_large<256, 256>(p, st);
  if (dqk == 256 && dv == 512) return launch_large<256, 512>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
