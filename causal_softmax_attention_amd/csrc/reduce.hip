// Log-sum-exp merge of split-K partials (ROCm/aiter PR #6660, third commit
// message and "Technical details": segment partials merged by a reduce, an
// empty partial with M = -inf weighs 0).
//
// One 256-thread workgroup per row.  Thread t = (split group sg, column
// chunk c) with CH = dv/4 chunks of 4 floats and SG = 256/CH groups: group
// sg sums splits sg, sg+SG, ... of chunk c, four splits' loads in flight at
// a time, so a row with a hundred splits costs a few memory latencies, not
// one per split.  Two passes: the max of m over the row's splits, then the
// exp(m_s - max) weighted sums of acc and l; the groups meet in LDS.  acc
// and l of an empty split (m = -inf) may be loaded (they are in range) but
// never enter a sum.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace

template <int CH, typename OutT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceParams p) {
  constexpr int SG = 256 / CH;
  constexpr int U = 4;                       // splits per group in flight
  __shared__ f32x4 part[SG][CH];
  __shared__ float red[2][4];
  const long row = blockIdx.x;
  const int t = threadIdx.x, sg = t / CH, c = t % CH, wave = t >> 6, lane = t & 63;

  int nsplit = p.num_splits;
  long first = row * (long)p.num_splits, step = 1;   // partial index of split 0, and stride
  if (p.seq_lens != nullptr) {
    const int tok = (int)(row / p.heads);
    if (tok >= p.cu_seqlens_q[p.num_requests]) return;   // whole workgroup
    int lo = 0, hi = p.num_requests;          // find r with cu[r] <= tok < cu[r+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_seqlens_q[mid] <= tok) lo = mid; else hi = mid;
    }
    if (p.balanced) {
      // the row's request: its pieces base .. base + n - 1 (published by the
      // partial kernel); piece k of head h is partial (base + k) * Hkv + h,
      // row t * (heads / Hkv) + head-in-group
      const int h = (int)(row % p.heads), grp = p.heads / p.Hkv;
      const int ui = (lo * p.Hkv + h / grp) * 2;
      const bool has_keys = p.seq_lens[lo] > 0;
      nsplit = has_keys ? p.unit_info[ui + 1] : 0;
      first = (has_keys ? ((long)p.unit_info[ui] * p.Hkv + h / grp) * p.rpu : 0) +
              (long)(tok - p.cu_seqlens_q[lo]) * grp + h % grp;
      step = (long)p.Hkv * p.rpu;
    } else {
      // only the segments that start at or before the row's own position
      // (the partial kernel writes exactly those)
      const int pos = p.seq_lens[lo] - p.cu_seqlens_q[lo + 1] + tok;   // L - qlen + t
      nsplit = pos < 0 ? 0 : min(nsplit, pos / p.split_len + 1);
    }
  }
  const float* m = p.m + first;
  const float* l = p.l + first;
  const float* acc = p.acc + first * p.dv + 4 * c;

  // ---- pass 1: max of m ----
  float M = -INFINITY;
  for (int s = t; s < nsplit; s += 256) M = fmaxf(M, m[s * step]);
  M = wave_max(M);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

  // ---- pass 2: weighted sums ----
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  if (M != -INFINITY) {
    for (int s0 = sg; s0 < nsplit; s0 += U * SG) {
      float ms[U], ls[U];
      f32x4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = min(s0 + u * SG, nsplit - 1);     // clamped: loads stay unconditional
        ms[u] = m[s * step];
        ls[u] = l[s * step];
        a[u] = *reinterpret_cast<const f32x4*>(acc + (long)s * step * p.dv);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u * SG < nsplit && ms[u] != -INFINITY) {
          const float w = expf(ms[u] - M);
          o += w * a[u];
          lsum += w * ls[u];
        }
      }
    }
  }
  part[sg][c] = o;
  // every thread of a split group saw the same splits: take l from chunk 0
  float lpart = (c == 0) ? lsum : 0.f;
  lpart = wave_sum(lpart);
  if (lane == 0) red[1][wave] = lpart;
  __syncthreads();
  const float Lsum = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  if (t < CH) {
    f32x4 sum = part[0][t];
#pragma unroll
    for (int j = 1; j < SG; ++j) sum += part[j][t];
    const float inv = (M == -INFINITY) ? 0.f : 1.0f / Lsum;
    OutT* out = reinterpret_cast<OutT*>(p.out) + row * p.dv + 4 * t;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (OutT)(sum[j] * inv);
  }
  if (p.lse != nullptr && t == 0)
    p.lse[row] = (M == -INFINITY) ? -INFINITY : M + logf(Lsum);
}

template <typename OutT>
static hipError_t launch_t(const ReduceParams& p, hipStream_t st) {
  dim3 grid((unsigned)p.rows), block(256);
  switch (p.dv) {
    case 64: splitk_reduce_kernel<16, OutT><<<grid, block, 0, st>>>(p); break;
    case 128: splitk_reduce_kernel<32, OutT><<<grid, block, 0, st>>>(p); break;
    case 256: splitk_reduce_kernel<64, OutT><<<grid, block, 0, st>>>(p); break;
    case 512: splitk_reduce_kernel<128, OutT><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  return p.out_fp32 ? launch_t<float>(p, st) : launch_t<bf16>(p, st);
}

}  // namespace attn
