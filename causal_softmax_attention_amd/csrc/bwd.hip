// Backward of packed variable-length causal attention for gfx950.
//
// Method (fla issue #1322): the gradients of the Description's feature set;
// the comment of Oct 3 (sink gradient accumulated directly as an fp32 sum of
// P * (dO V^T) times the negative sink probability, reduced over queries,
// instead of through delta computed from the rounded output); the comment of
// Oct 5 (dQ fused into the dK/dV pass so each score and dP tile is computed
// once, dQ partials added into a zero-initialised fp32 buffer and converted
// to the input dtype afterwards; gate and sink partials as fp32 reductions).
//
// Launches (plus the gate prefix scan shared with the forward):
//   bwd_pre   delta_i = sum_d fp32(O) fp32(dO) and the row term G2 - lse
//             log2(e), head-major (with a dS store also psink_i); zero
//             dq_acc, dG, dsink
//   then either the deterministic two-pass kernels (bwd2.h, bwd_large.h),
//   or bwd_fused (bwd_fused.h: dQ through fp32 atomics, pre-reduced over
//   the workgroup's keys) followed by
//   bwd_post  dq = bf16(dq_acc); dg = reverse cumsum of dG per sequence
#include "bwd_fused.h"
#include "common.h"
#include "kernels.h"

namespace attn {

// ---------------------------------------------------------------------------
// delta = sum_d O[row, d] * dO[row, d] in fp32 (row = token * Hq + head),
// stored head-major [Hq, T]; for the two-pass kernels also the row term
// G2 - lse * log2(e), head-major, so that a tile's rows are contiguous.
// DV/8 lanes per row, 16 bytes of O and of dO per lane, so a wave streams
// whole 256-byte rows; also zeroes the fused path's dQ accumulator and the
// gate / sink gradient accumulators.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = DV / 8;                 // lanes per row
  constexpr int RPB = 256 / LPR;              // rows per workgroup
  const int t = threadIdx.x, sub = t % LPR;
  const long row = (long)blockIdx.x * RPB + t / LPR;
  if (blockIdx.x == 0 && p.dsink_acc != nullptr)
    for (int h = t; h < p.Hq; h += 256) p.dsink_acc[h] = 0.f;
  if (row >= (long)p.T * p.Hq) return;
  // O is read once, here (non-temporal); dO is read again by both passes
  const bf16x8 o = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
      reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.o) + row * DV + 8 * sub)));
  const bf16x8 d = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(p.dO) + row * DV + 8 * sub);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)o[j] * (float)d[j];
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (sub == 0) {
    const long tok = row / p.Hq;
    const long hm = (row - tok * p.Hq) * p.T + tok;   // head-major index
    p.delta[hm] = s;
    if (p.rowt != nullptr) p.rowt[hm] = (p.G2 != nullptr ? p.G2[hm] : 0.f) - p.lse[row] * kLog2e;
    if (p.psink != nullptr) p.psink[hm] = fast_exp2((p.sink[row - tok * p.Hq] - p.lse[row]) * kLog2e);
    if (p.dG != nullptr) p.dG[row] = 0.f;
  }
  if (p.dq_acc != nullptr) {
    float* dqa = p.dq_acc + row * DQK;
    for (int j = sub; j < DQK / 4; j += LPR) *reinterpret_cast<f32x4*>(dqa + 4 * j) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                             bf16* __restrict__ dq, long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = reinterpret_cast<const f32x4*>(acc)[i];
  reinterpret_cast<bf16x4*>(dq)[i] = to_bf16x4(x);
}

// dg[t, h] = sum over s >= t within t's sequence of dG[s, h] (a reverse
// scan): one workgroup per (head, sequence).  dG[t, h] = a[t, h] - b[t, h]
// (b may be null), both read at t * st_t + h * st_h (head-major partials of
// the two-pass path, token-major accumulator of the fused one).
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* __restrict__ a_,
                                                        const float* __restrict__ b_,
                                                        const int32_t* __restrict__ cu,
                                                        float* __restrict__ dg, int Hq, long st_t,
                                                        long st_h) {
  const int h = blockIdx.x, n = blockIdx.y;
  const int a = cu[n], L = cu[n + 1] - a;
  if (L <= 0) return;
  const long base = (long)a * st_t + h * st_h;
  float* out = dg + (long)a * Hq + h;
  // scan order q runs from the sequence's last token to its first
  block_scan_256(
      L,
      [&](int q) {
        const long i = base + (long)(L - 1 - q) * st_t;
        return b_ ? a_[i] - b_[i] : a_[i];
      },
      [&](int q, float v) { out[(long)(L - 1 - q) * Hq] = v; });
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* x, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

hipError_t launch_fill_zero(float* x, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_zero_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(x, n);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_fused_t(const BwdParams& p, hipStream_t st) {
  const long rows = (long)p.T * p.Hq;
  hipError_t e = launch_fused_kernel<DQK, DV>(p, st);   // bwd_fused.h
  if (e != hipSuccess) return e;
  const long n4 = rows * DQK / 4;
  bwd_dq_convert_kernel<DQK><<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(
      p.dq_acc, reinterpret_cast<bf16*>(p.dq), n4);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.dg != nullptr) {
    gate_grad_kernel<<<dim3(p.Hq, p.num_seqs), 256, 0, st>>>(p.dG, nullptr, p.cu, p.dg, p.Hq, p.Hq, 1);
    e = hipGetLastError();
  }
  return e;
}

template <int DQK, int DV>
static hipError_t launch_bwd_t(const BwdParams& p, bool fused, hipStream_t st) {
  const long rows = (long)p.T * p.Hq;
  constexpr int RPB = 256 / (DV / 8);
  bwd_pre_kernel<DQK, DV><<<dim3((unsigned)((rows + RPB - 1) / RPB)), 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (DQK <= 128) {   // the fused-dQ path covers query/key head dims up to 128
    if (fused) return launch_fused_t<DQK, DV>(p, st);
  }
  e = launch_bwd_two_pass(p, DQK, DV, st);
  if (e != hipSuccess) return e;
  if (p.dg != nullptr) {
    gate_grad_kernel<<<dim3(p.Hq, p.num_seqs), 256, 0, st>>>(p.dGrow, p.dGcol, p.cu, p.dg, p.Hq, 1, p.T);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(const BwdParams& p, int dqk, int dv, bool fused, hipStream_t st) {
  if (p.num_seqs == 0 || p.T == 0 || p.max_seqlen == 0) {
    return hipSuccess;
  }
  switch (dqk * 1000 + dv) {
    case 64064: return launch_bwd_t<64, 64>(p, fused, st);
    case 64128: return launch_bwd_t<64, 128>(p, fused, st);
    case 64256: return launch_bwd_t<64, 256>(p, fused, st);
    case 64512: return launch_bwd_t<64, 512>(p, fused, st);
    case 128064: return launch_bwd_t<128, 64>(p, fused, st);
    case 128128: return launch_bwd_t<128, 128>(p, fused, st);
    case 128256: return launch_bwd_t<128, 256>(p, fused, st);
    case 128512: return launch_bwd_t<128, 512>(p, fused, st);
    case 256064: return launch_bwd_t<256, 64>(p, fused, st);
    case 256128: return launch_bwd_t<256, 128>(p, fused, st);
    case 256256: return launch_bwd_t<256, 256>(p, fused, st);
    case 256512: return launch_bwd_t<256, 512>(p, fused, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
