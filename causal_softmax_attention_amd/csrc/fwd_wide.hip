// Forward for query/key head dim 256 (value head dims 64 to 512); the
// kernel is in fwd_large.h.  Kept apart from fwd.hip: its O accumulators
// keep the default AGPR allocation, which the head-dim 64 / 128 kernels turn
// off.
#include "fwd_large.h"

namespace attn {

hipError_t launch_fwd_wide(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk != 256) return hipErrorInvalidValue;
  switch (dv) {
    case 64: return launch_large<256, 64>(p, st);
    case 128: return launch_large<256, 128>(p, st);
    case 256: return launch_large<256, 256>(p, st);
    case 512: return launch_large<256, 512>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
