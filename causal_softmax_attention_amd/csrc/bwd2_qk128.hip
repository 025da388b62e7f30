// Two-pass backward instantiations for query/key head dim 128 (the kernels
// are in bwd2.h).
#include "bwd2.h"

namespace attn {

hipError_t launch_bwd_two_pass_qk128(const BwdParams& p, int dv, hipStream_t st) {
  return launch_bwd_two_pass_qk<128>(p, dv, st);
}

}  // namespace attn
