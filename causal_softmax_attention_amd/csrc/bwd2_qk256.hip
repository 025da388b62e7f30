// Two-pass backward instantiations for query/key head dim 256 (the kernels
// are in bwd2.h).
#include "bwd2.h"

namespace attn {

hipError_t launch_bwd_two_pass_qk256(const BwdParams& p, int dv, hipStream_t st) {
  return launch_bwd_two_pass_qk<256>(p, dv, st);
}

}  // namespace attn
