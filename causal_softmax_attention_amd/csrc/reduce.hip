// Log-sum-exp merge of split-K partials (ROCm/aiter PR #6660, third commit
// message and "Technical details": segment partials merged by a reduce, an
// empty partial with M = -inf weighs 0).
//
// One workgroup per row.  Thread t = (split group sg, column chunk c) with
// CH = dv/4 chunks of 4 floats and SG split groups (SG = 256/CH when a row
// holds many splits, 2 when it holds a few: then a workgroup is one wave
// for dv = 128 and every row's workgroup is resident at once): group
// sg sums splits sg, sg+SG, ... of chunk c, four splits' loads in flight at
// a time, so a row with a hundred splits costs a few memory latencies, not
// one per split.  One pass: each group keeps its own running max over its
// splits (rescaling what it holds when the max rises); the groups meet in
// LDS, weighted by exp(group max - row max).  acc and l of an empty split
// (m = -inf) may be loaded (they are in range) but never enter a sum.
#include "common.h"
#include "kernels.h"

namespace attn {


template <int CH, int SG, typename OutT>
__global__ __launch_bounds__(CH * SG) void splitk_reduce_kernel(ReduceParams p) {
  static_assert(CH * SG <= 256 && (CH * SG) % 64 == 0, "block of whole waves, at most 256 threads");
  constexpr int U = 4;                       // splits per group in flight
  __shared__ f32x4 part[SG][CH];
  __shared__ float gm[SG], gl[SG];        // each split group's max and weighted l
  const long row = blockIdx.x;
  const int t = threadIdx.x, sg = t / CH, c = t % CH, lane = t & 63;

  int nsplit = p.num_splits;
  long first = row * (long)p.num_splits, step = 1;   // partial index of split 0, and stride
  if (p.seq_lens != nullptr) {
    const int tok = (int)(row / p.heads);
    // the row's request r: the last with cu[r] <= tok (a request with no
    // tokens shares its start with the next one), 64 starts per wave load
    // instead of a chain of dependent loads
    const int T = p.cu_seqlens_q[p.num_requests];
    int lo = 0;
    for (int c0 = 0; c0 < p.num_requests; c0 += 64) {
      const int i = c0 + lane;
      const unsigned long long le = __ballot(i < p.num_requests && p.cu_seqlens_q[i] <= tok);
      if (le != 0) lo = c0 + 63 - __builtin_clzll(le);
      if (le != ~0ull) break;
    }
    if (tok >= T) return;                     // whole workgroup
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

  // ---- one pass: each split group merges its splits under its own running
  // max (m, l and acc loaded together); the groups meet in LDS ----
  float Mg = -INFINITY;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
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
        if (ms[u] > Mg) {                 // rescale what this group holds
          const float f = expf(Mg - ms[u]);
          o *= f;
          lsum *= f;
          Mg = ms[u];
        }
        const float w = expf(ms[u] - Mg);
        o += w * a[u];
        lsum += w * ls[u];
      }
    }
  }
  part[sg][c] = o;
  if (c == 0) {                           // every thread of a group saw the same splits
    gm[sg] = Mg;
    gl[sg] = lsum;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < SG; ++j) M = fmaxf(M, gm[j]);
  float Lsum = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < SG; ++j)
      if (gm[j] != -INFINITY) Lsum += gl[j] * expf(gm[j] - M);
  }
  if (t < CH) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int j = 0; j < SG; ++j)
        if (gm[j] != -INFINITY) sum += part[j][t] * expf(gm[j] - M);
    }
    const float inv = (M == -INFINITY) ? 0.f : 1.0f / Lsum;
    OutT* out = reinterpret_cast<OutT*>(p.out) + row * p.dv + 4 * t;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (OutT)(sum[j] * inv);
  }
  if (p.lse != nullptr && t == 0)
    p.lse[row] = (M == -INFINITY) ? -INFINITY : M + logf(Lsum);
}

template <int CH, typename OutT>
static void launch_ch(const ReduceParams& p, bool few, hipStream_t st) {
  constexpr int SG_MANY = 256 / CH, SG_FEW = CH >= 32 ? 2 : 4;
  const dim3 grid((unsigned)p.rows);
  if (few)
    splitk_reduce_kernel<CH, SG_FEW, OutT><<<grid, dim3(CH * SG_FEW), 0, st>>>(p);
  else
    splitk_reduce_kernel<CH, SG_MANY, OutT><<<grid, dim3(CH * SG_MANY), 0, st>>>(p);
}

template <typename OutT>
static hipError_t launch_t(const ReduceParams& p, hipStream_t st) {
  // a few splits per row: two split groups (U = 4 loads in flight each)
  // cover up to 8 splits in one round of loads
  const int splits = p.splits_hint > 0 ? p.splits_hint : p.num_splits;
  const bool few = splits <= 8;
  switch (p.dv) {
    case 64: launch_ch<16, OutT>(p, few, st); break;
    case 128: launch_ch<32, OutT>(p, few, st); break;
    case 256: launch_ch<64, OutT>(p, false, st); break;
    case 512: launch_ch<128, OutT>(p, false, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  return p.out_fp32 ? launch_t<float>(p, st) : launch_t<bf16>(p, st);
}

}  // namespace attn
