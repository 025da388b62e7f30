// Forward for query/key head dim 128 with value head dim 256 or 512; the
// kernel is in fwd_large.h.
#include "fwd_large.h"

namespace attn {

hipError_t launch_fwd_large_qk128(const FwdParams& p, int dv, hipStream_t st) {
  if (dv == 256) return launch_large<128, 256>(p, st);
  if (dv == 512) return launch_large<128, 512>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
