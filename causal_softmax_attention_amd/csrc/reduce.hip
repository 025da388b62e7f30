// Log-sum-exp merge of split-K partials (ROCm/aiter PR #6660, third commit
// message and "Technical details": segment partials merged by a reduce, an
// empty partial with M = -inf weighs 0).
//
// One wavefront per row; lane l owns columns [l*V, l*V+V) with V = Dv/64.
// Two passes over the row's splits: the max of m, then the weighted sums.
// acc and l of an empty split (m = -inf) are never read.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int V, typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;

  int nsplit = p.num_splits;
  if (p.seq_lens != nullptr) {
    // Decode rows: only the segments that exist for this row's request.
    const int tok = (int)(row / p.heads);
    if (tok >= p.cu_seqlens_q[p.num_requests]) return;   // past the last query token
    int lo = 0, hi = p.num_requests;          // find r with cu[r] <= tok < cu[r+1]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (p.cu_seqlens_q[mid] <= tok) lo = mid; else hi = mid;
    }
    const int L = p.seq_lens[lo];
    nsplit = min(nsplit, (L + p.split_len - 1) / p.split_len);
  }
  const float* m = p.m + row * p.num_splits;
  const float* l = p.l + row * p.num_splits;
  const float* acc = p.acc + row * (long)p.num_splits * p.dv + lane * V;

  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, m[s]);

  float o[V];
#pragma unroll
  for (int j = 0; j < V; ++j) o[j] = 0.f;
  float Lsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float ms = m[s];
      if (ms == -INFINITY) continue;
      const float w = expf(ms - M);
      Lsum += w * l[s];
      const float* a = acc + (long)s * p.dv;
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] += w * a[j];
    }
    const float inv = 1.0f / Lsum;
#pragma unroll
    for (int j = 0; j < V; ++j) o[j] *= inv;
  }
  OutT* out = reinterpret_cast<OutT*>(p.out) + row * p.dv + lane * V;
#pragma unroll
  for (int j = 0; j < V; ++j) out[j] = (OutT)o[j];
  if (p.lse != nullptr && lane == 0)
    p.lse[row] = (M == -INFINITY) ? -INFINITY : M + logf(Lsum);
}

template <typename OutT>
static hipError_t launch_t(const ReduceParams& p, hipStream_t st) {
  dim3 grid((unsigned)((p.rows + 3) / 4)), block(256);
  switch (p.dv / 64) {
    case 1: splitk_reduce_kernel<1, OutT><<<grid, block, 0, st>>>(p); break;
    case 2: splitk_reduce_kernel<2, OutT><<<grid, block, 0, st>>>(p); break;
    case 4: splitk_reduce_kernel<4, OutT><<<grid, block, 0, st>>>(p); break;
    case 8: splitk_reduce_kernel<8, OutT><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  return p.out_fp32 ? launch_t<float>(p, st) : launch_t<bf16>(p, st);
}

}  // namespace attn
