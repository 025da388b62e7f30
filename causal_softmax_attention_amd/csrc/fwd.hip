// Packed variable-length causal attention forward for gfx950.
//
// Method (fla issue #1322, Description): causal softmax attention over
// packed sequences with MHA/GQA/MQA, unequal q/k and v head dims, a
// logarithmic gate bias G_i - G_j (G = per-sequence inclusive cumsum of the
// log gates), a sliding window and a per-head sink logit that adds mass to
// the softmax denominator but carries no value.  Scores are accumulated in
// fp32 from bf16 operands; probabilities enter PV as bf16; O is rounded to
// bf16 at the end and lse is kept in fp32.
//
// gfx950 mapping
//  * Tile schedule: grid (query head, sequence, query tile), the query-tile
//    index reversed so the longest tiles are dispatched first; tiles past a
//    sequence's end exit at once.  A tile of BM query rows visits the KV
//    range [max(0, i0 - W + 1), min(L, i0 + BM)); tiles outside the causal
//    or window band are never loaded.
//  * Four wavefronts per workgroup, RW query rows each; Q stays in
//    registers as the B operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16),
//    so each lane owns one query row of every 16-row block and a row's
//    max / sum needs only two cross-lane steps.
//  * K and V tiles of BN keys are staged in LDS (row strides padded against
//    bank conflicts); V^T operands come from ds_read_b64_tr_b16, so P leaves
//    the score registers straight into the PV MFMA with no shuffle.
//  * Online softmax in base 2: scores are scaled by softmax_scale*log2(e)
//    and the gate prefix is stored pre-multiplied by log2(e); the running
//    max starts at the sink logit with l = 1.  Masking is applied only on
//    tiles that cross the diagonal, the window edge or the sequence end.
#include "common.h"
#include "kernels.h"

#ifndef FWD_RW_SMALL
#define FWD_RW_SMALL 16
#endif
#ifndef FWD_BN_SMALL
#define FWD_BN_SMALL 64
#endif

namespace attn {

// ---------------------------------------------------------------------------
// Gate prefix: G2[t, h] = log2(e) * sum of g[s, h] over s from the start of
// t's sequence to t.  One workgroup per (sequence, head); each thread scans a
// contiguous chunk, chunk totals are scanned in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_prefix_kernel(const float* __restrict__ g,
                                                          const int32_t* __restrict__ cu,
                                                          float* __restrict__ G2, int Hq) {
  const int h = blockIdx.x, n = blockIdx.y;
  const int a = cu[n], L = cu[n + 1] - a;
  if (L <= 0) return;
  const int chunk = (L + 255) / 256;
  const int t0 = threadIdx.x * chunk;
  const int t1 = min(L, t0 + chunk);
  float s = 0.f;
  for (int t = t0; t < t1; ++t) s += g[(long)(a + t) * Hq + h];
  __shared__ float part[256];
  part[threadIdx.x] = s;
  __syncthreads();
  // inclusive Hillis-Steele scan of the 256 chunk totals
  for (int off = 1; off < 256; off <<= 1) {
    float v = threadIdx.x >= off ? part[threadIdx.x - off] : 0.f;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  float run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0.f;
  for (int t = t0; t < t1; ++t) {
    run += g[(long)(a + t) * Hq + h];
    G2[(long)(a + t) * Hq + h] = run * kLog2e;
  }
}

hipError_t launch_gate_prefix(const float* g, const int32_t* cu, float* G2, int num_seqs,
                              int T, int Hq, hipStream_t st) {
  if (num_seqs == 0 || T == 0) return hipSuccess;
  gate_prefix_kernel<<<dim3(Hq, num_seqs), 256, 0, st>>>(g, cu, G2, Hq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2);
// map block x so that the query heads of one KV group land on one XCD.
__device__ __forceinline__ int xcd_head(int x, int Hq) {
  if (Hq % 8 != 0) return x;
  return (x % 8) * (Hq / 8) + x / 8;
}

template <int DQK, int DV, int RW, int BN, bool GATED>
__global__ __launch_bounds__(256) void fwd_kernel(FwdParams p) {
  constexpr int BM = 4 * RW;
  constexpr int RBW = RW / 16;       // 16-row blocks per wave
  constexpr int KB = BN / 16;        // 16-key blocks per tile
  constexpr int KS = DQK / 32;       // k-steps over d_qk
  constexpr int DB = DV / 16;        // 16-wide output column blocks
  constexpr int KROW = DQK + 8;      // LDS row strides (elements)
  constexpr int VROW = DV + 16;
  constexpr int KCH = BN * DQK / 8 / 256;   // 16-byte chunks per thread per tile
  constexpr int VCH = BN * DV / 8 / 256;
  static_assert(KB % 2 == 0, "PV consumes keys in pairs of 16-key blocks");
  static_assert(KCH * 256 * 8 == BN * DQK && VCH * 256 * 8 == BN * DV, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2][BN * VROW];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][BN];

  const int h = xcd_head(blockIdx.x, p.Hq), n = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int i0 = tile * BM;
  if (i0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int kvh = h / grp;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
  constexpr bool gated = GATED;
  const float c = p.scale_log2;

  const int r0 = i0 + wave * RW;                 // first row of this wave
  const int r_last = min(r0 + RW, L) - 1;        // last real row (may be < r0)

  // ---- Q operand and per-row state (running max m is kept without the
  //      row's own gate term gq, which is constant along the row) ----
  bf16x8 qop[RBW][KS];
  float gq[RBW], m_run[RBW], l_run[RBW];
  f32x4 oacc[RBW][DB];
  const float sink2 = p.sink ? p.sink[h] * kLog2e : kNegBig;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = r0 + rb * 16 + li;
    if (row < L) {
      const bf16* qp = reinterpret_cast<const bf16*>(p.q) + ((long)(seq0 + row) * p.Hq + h) * DQK + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
      gq[rb] = gated ? p.G2[(long)(seq0 + row) * p.Hq + h] : 0.f;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = bf16x8{};
      gq[rb] = 0.f;
    }
    m_run[rb] = p.sink ? sink2 - gq[rb] : kNegBig;
    l_run[rb] = p.sink ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BM);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long)seq0 * p.Hkv + kvh) * DQK;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long)seq0 * p.Hkv + kvh) * DV;
  const long kstride = (long)p.Hkv * DQK, vstride = (long)p.Hkv * DV;

  // ---- register staging of one K/V tile (global -> regs -> LDS) ----
  i32x4 kreg[KCH], vreg[VCH];
  float gkreg = 0.f;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DQK / 8), col = (ch % (DQK / 8)) * 8;
      const int key = min(j0 + kr, L - 1);       // rows past the end: any valid row
      kreg[cc] = *reinterpret_cast<const i32x4*>(kbase + (long)key * kstride + col);
    }
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DV / 8), col = (ch % (DV / 8)) * 8;
      const int key = min(j0 + kr, L - 1);
      vreg[cc] = *reinterpret_cast<const i32x4*>(vbase + (long)key * vstride + col);
    }
    if (gated && tid < BN) gkreg = p.G2[(long)(seq0 + min(j0 + tid, L - 1)) * p.Hq + h];
  };
  auto stash = [&](int buf, int j0) {
    const i32x4 z = {0, 0, 0, 0};
    const bool tail = j0 + BN > L;               // zero-fill rows past the end (last tile only)
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DQK / 8), col = (ch % (DQK / 8)) * 8;
      *reinterpret_cast<i32x4*>(&k_lds[buf][kr * KROW + col]) = (tail && j0 + kr >= L) ? z : kreg[cc];
    }
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DV / 8), col = (ch % (DV / 8)) * 8;
      *reinterpret_cast<i32x4*>(&v_lds[buf][kr * VROW + col]) = (tail && j0 + kr >= L) ? z : vreg[cc];
    }
    if (gated && tid < BN) gk_lds[buf][tid] = gkreg;
  };

  fetch(t_begin * BN);
  stash(0, t_begin * BN);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int j0 = t * BN;
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    // Unconditional (addresses are clamped in range) so the compiler does not
    // drain the loads at a branch join before the math below.
    fetch(j0 + BN);

    // No branch around the math: a tile that is wholly masked for this
    // wave's rows goes through the masked path and contributes zeros.  (A
    // branch here makes the compiler shuttle every accumulator between
    // AGPRs and VGPRs on each iteration.)
    {
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + RW - 1);
      const bf16* kl = k_lds[buf];
      const bf16* vl = v_lds[buf];
      // ---- S^T = K Q^T ----
      f32x4 sc[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = lds_read8(kl + (kb * 16 + li) * KROW + ks * 32 + 8 * g);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = mfma16x16x32(a, qop[rb][ks], sc[kb][rb]);
        }
      }
      // ---- y = s*c - gk (base 2, without the row's gate term) ----
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 gk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(&gk_lds[buf][kb * 16 + 4 * g]);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[kb][rb][i] = GATED ? __builtin_fmaf(sc[kb][rb][i], c, -gk[i]) : sc[kb][rb][i] * c;
      }
      // ---- mask, only on tiles crossing the diagonal, window edge or end ----
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            const int row = r0 + rb * 16 + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = j0 + kb * 16 + 4 * g + i;
              const bool vis = key <= row && key < L && (W <= 0 || row - key < W);
              sc[kb][rb][i] = vis ? sc[kb][rb][i] : -INFINITY;
            }
          }
      }
      // ---- online softmax with lazy rescale ----
      bf16x4 pb[KB][RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          mx = fmaxf(mx, fmaxf(fmaxf(sc[kb][rb][0], sc[kb][rb][1]), fmaxf(sc[kb][rb][2], sc[kb][rb][3])));
        mx = xgroup_max(mx);
        if (__builtin_expect(__any(mx > m_run[rb] + kRescaleSlack), 0)) {
          const float m_new = fmaxf(m_run[rb], mx);
          const float alpha = fast_exp2(m_run[rb] - m_new);
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
          m_run[rb] = m_new;
        }
        const float mr = m_run[rb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          f32x4 e;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = fast_exp2(sc[kb][rb][i] - mr);
            rs += e[i];
          }
          pb[kb][rb] = to_bf16x4(e);
        }
        l_run[rb] += xgroup_sum(rs);
      }
      // ---- O^T += V^T P^T, 32 keys per MFMA ----
#pragma unroll
      for (int kp = 0; kp < KB / 2; ++kp) {
        const int mm = li >> 2, c4 = li & 3;
        const bf16* vr0 = vl + (kp * 32 + 4 * g + mm) * VROW + 4 * c4;
        const bf16* vr1 = vl + (kp * 32 + 16 + 4 * g + mm) * VROW + 4 * c4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = concat(lds_read_tr16(vr0 + db * 16), lds_read_tr16(vr1 + db * 16));
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            oacc[rb][db] = mfma16x16x32(a, concat(pb[2 * kp][rb], pb[2 * kp + 1][rb]), oacc[rb][db]);
        }
      }
    }
    if (more) stash(buf ^ 1, j0 + BN);
    __syncthreads();
  }

  // ---- finalize: O = acc / l, lse = ln 2 * (m + gq + log2 l) ----
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = r0 + rb * 16 + li;
    if (row >= L) continue;
    const float inv = 1.0f / l_run[rb];
    bf16* op = reinterpret_cast<bf16*>(p.o) + ((long)(seq0 + row) * p.Hq + h) * DV + 4 * g;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 x = oacc[rb][db] * inv;
      *reinterpret_cast<bf16x4*>(op + db * 16) = to_bf16x4(x);
    }
    if (g == 0)
      p.lse[(long)(seq0 + row) * p.Hq + h] = (m_run[rb] + gq[rb] + fast_log2(l_run[rb])) * kLn2;
  }
}

template <int DQK, int DV, int RW, int BN>
static hipError_t launch_cfg(const FwdParams& p, hipStream_t st) {
  constexpr int BM = 4 * RW;
  const int tiles = (p.max_seqlen + BM - 1) / BM;
  dim3 grid(p.Hq, p.num_seqs, tiles), block(256);
  if (p.G2 != nullptr)
    fwd_kernel<DQK, DV, RW, BN, true><<<grid, block, 0, st>>>(p);
  else
    fwd_kernel<DQK, DV, RW, BN, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (p.num_seqs == 0 || p.T == 0 || p.max_seqlen == 0) return hipSuccess;
  if (dqk == 64 && dv == 64) return launch_cfg<64, 64, FWD_RW_SMALL, FWD_BN_SMALL>(p, st);
  if (dqk == 128 && dv == 128) return launch_cfg<128, 128, FWD_RW_SMALL, FWD_BN_SMALL>(p, st);
  if (dqk == 256 && dv == 256) return launch_cfg<256, 256, 16, 32>(p, st);
  if (dqk == 256 && dv == 512) return launch_cfg<256, 512, 16, 32>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
