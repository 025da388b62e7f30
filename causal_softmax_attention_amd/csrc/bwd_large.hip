// dK/dV and dQ passes of the two-pass backward for query/key head dim 256
// with value head dims 256 and 512 (the kernels are in bwd_large.h).  Kept
// apart from the other backward kernels: their accumulators may live in
// AGPRs, which those kernels' translation units turn off.
#include "bwd_large.h"

namespace attn {

hipError_t launch_dkdv_large(const BwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 256 && dv == 256) return launch_dkdv_large_t<256, 256>(p, st);
  if (dqk == 256 && dv == 512) return launch_dkdv_large_t<256, 512>(p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_dq_large(const BwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 256 && dv == 256) return launch_dq_large_t<256, 256>(p, st);
  if (dqk == 256 && dv == 512) return launch_dq_large_t<256, 512>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
