// Forward entry points: the gate prefix, the dispatch over head dims and the
// kernels for query/key and value head dims of 64 or 128 (the kernel itself
// is in fwd_pipe.h).  The other pairs use the large-head kernel in
// fwd_large.h, instantiated in fwd_wide.hip (query/key head dim 256) and
// fwd_large_qk64.hip / fwd_large_qk128.hip (value head dim 256 or 512),
// which are built with different register allocation options.
#include "fwd_pipe.h"

namespace attn {

// ---------------------------------------------------------------------------
// Gate prefix: G2[h, t] = log2(e) * sum of g[s, h] over s from the start of
// t's sequence to t.  Head-major, so that the gate terms of a tile's
// consecutive keys (or rows) of one head are contiguous.  One workgroup per
// (head, sequence); each thread scans a contiguous chunk, chunk totals are
// scanned in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_prefix_kernel(const float* __restrict__ g,
                                                          const int32_t* __restrict__ cu,
                                                          float* __restrict__ G2, int Hq, int T) {
  const int h = blockIdx.x, n = blockIdx.y;
  const int a = cu[n], L = cu[n + 1] - a;
  if (L <= 0) return;
  const float* gs = g + (long)a * Hq + h;
  float* out = G2 + (long)h * T + a;
  block_scan_256(L, [&](int t) { return gs[(long)t * Hq]; }, [&](int t, float v) { out[t] = v * kLog2e; });
}

hipError_t launch_gate_prefix(const float* g, const int32_t* cu, float* G2, int num_seqs,
                              int T, int Hq, hipStream_t st) {
  if (num_seqs == 0 || T == 0) return hipSuccess;
  gate_prefix_kernel<<<dim3(Hq, num_seqs), 256, 0, st>>>(g, cu, G2, Hq, T);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (p.num_seqs == 0 || p.T == 0 || p.max_seqlen == 0) return hipSuccess;
  if (dqk == 64 && dv == 64) return launch_pipe<64, 64>(p, st);
  if (dqk == 64 && dv == 128) return launch_pipe<64, 128>(p, st);
  if (dqk == 128 && dv == 64) return launch_pipe<128, 64>(p, st);
  if (dqk == 128 && dv == 128) return launch_pipe<128, 128>(p, st);
  if (dqk == 64) return launch_fwd_large_qk64(p, dv, st);
  if (dqk == 128) return launch_fwd_large_qk128(p, dv, st);
  if (dqk == 256) return launch_fwd_wide(p, dqk, dv, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
