// Two-pass backward: the sink-gradient reduction, the dispatch over head
// dims, and the instantiations for query/key head dim 64 (the kernels are in
// bwd2.h).
#include "bwd2.h"

namespace attn {

// dsink[h] = -sum over all tokens of sink_rows[h, t] (fixed order).
__global__ __launch_bounds__(1024) void sink_reduce_kernel(const float* __restrict__ rows, float* __restrict__ dsink,
                                                           int T, int Hq) {
  // rows head-major [Hq, T]: thread t sums its contiguous share, 16 values
  // per round held in registers (one memory latency per round; one round up
  // to 16K tokens)
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* r = rows + (long)h * T;
  const int share = (T + 1023) / 1024;
  const int t0 = tid * share, t1 = min(T, t0 + share);
  float s = 0.f;
  for (int b0 = t0; b0 < t1; b0 += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = b0 + j < t1 ? r[b0 + j] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  __shared__ float part[1024];
  part[tid] = s;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  if (tid == 0) dsink[h] = -part[0];
}

hipError_t launch_sink_reduce(const BwdParams& p, hipStream_t st) {
  sink_reduce_kernel<<<dim3(p.Hq), 1024, 0, st>>>(p.sink_rows, p.dsink_acc, p.T, p.Hq);
  return hipGetLastError();
}

hipError_t launch_bwd_two_pass_qk64(const BwdParams& p, int dv, hipStream_t st) {
  return launch_bwd_two_pass_qk<64>(p, dv, st);
}

hipError_t launch_bwd_two_pass(const BwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 64) return launch_bwd_two_pass_qk64(p, dv, st);
  if (dqk == 128) return launch_bwd_two_pass_qk128(p, dv, st);
  if (dqk == 256) return launch_bwd_two_pass_qk256(p, dv, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
