// Deterministic two-pass backward for gfx950 (no atomics anywhere).
//
// The fla issue #1322 comment of Oct 5 keeps a two-pass backward for
// deterministic mode and for shapes the fused-dQ kernel does not cover.
// Here:
//   bwd_dkdv  KV-major: one workgroup per (4*KW keys, KV head, sequence),
//             each wavefront owning KW keys; dK^T, dV^T accumulate in
//             registers over the group's query heads and the 32-row query
//             tiles that see the keys.  Column sums of dS for the gate
//             gradient are complete per (key, head) in one wavefront, so
//             they are stored, not added.
//   bwd_dq    Q-major (the forward's structure): Q and dO rows stay in
//             registers, K/V tiles stream through LDS; dQ^T accumulates in
//             registers from K^T (ds_read_b64_tr_b16) times dS^T.  Row sums of
//             dS (gate gradient) and sum_j P dP (sink gradient, Oct 3 comment:
//             a direct fp32 sum from the recomputed probabilities) are
//             complete per row and stored.
// Both recompute S = QK^T and dP = dO V^T; dQ costs those two products
// again instead of fp32 atomics.
#include "common.h"
#include "kernels.h"

#ifndef BWD_KW_SMALL
#define BWD_KW_SMALL 16
#endif
#ifndef BWD_RW_SMALL
#define BWD_RW_SMALL 16
#endif

namespace attn {

__device__ __forceinline__ int xcd_remap(int x, int n) {
  // consecutive logical indices -> same XCD (blocks go round-robin over 8)
  if (n % 8 != 0) return x;
  return (x % 8) * (n / 8) + x / 8;
}

// ---------------------------------------------------------------------------
// PF: fetch the next query tile into registers during the current one
// (off for the largest heads, where those registers are not available).
template <int DQK, int DV, int KW, bool PF, bool GATED>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int RQ = 32;              // query rows per tile
  constexpr int KBW = KW / 16;        // 16-key blocks per wave
  constexpr int BNW = 4 * KW;         // keys per workgroup
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int DBQ = DQK / 16, DBV = DV / 16;
  constexpr int QROW = DQK + 8, OROW = DV + 16;
  constexpr int QCH = RQ * DQK / 8 / 256, OCH = RQ * DV / 8 / 256;   // 16-byte chunks per thread
  static_assert(QCH * 256 * 8 == RQ * DQK && OCH * 256 * 8 == RQ * DV, "tile must split evenly");
  constexpr int NB = PF ? 2 : 1;
  __shared__ __attribute__((aligned(16))) bf16 q_lds[NB][RQ * QROW];
  __shared__ __attribute__((aligned(16))) bf16 do_lds[NB][RQ * OROW];
  __shared__ __attribute__((aligned(16))) float lse_lds[NB][RQ], delta_lds[NB][RQ], gq_lds[NB][RQ];

  const int kvh = xcd_remap(blockIdx.x, p.Hkv), n = blockIdx.y, ktile = blockIdx.z;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int j0 = ktile * BNW;
  if (j0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
  constexpr bool gated = GATED;
  const int jw = j0 + wave * KW;

  bf16x8 kop[KBW][KSQ], vop[KBW][KSV];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int key = jw + kb * 16 + li;
    const bool ok = key < L;
    const bf16* kp = reinterpret_cast<const bf16*>(p.k) + ((long)(seq0 + min(key, L - 1)) * p.Hkv + kvh) * DQK + 8 * g;
    const bf16* vp = reinterpret_cast<const bf16*>(p.v) + ((long)(seq0 + min(key, L - 1)) * p.Hkv + kvh) * DV + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) kop[kb][ks] = ok ? *reinterpret_cast<const bf16x8*>(kp + 32 * ks) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) vop[kb][ks] = ok ? *reinterpret_cast<const bf16x8*>(vp + 32 * ks) : bf16x8{};
  }
  f32x4 dk_acc[KBW][DBQ], dv_acc[KBW][DBV];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
    for (int db = 0; db < DBQ; ++db) dk_acc[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DBV; ++db) dv_acc[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Flattened iteration over (query head of the group, 32-row query tile);
  // tile it+1 is fetched into registers while tile it is computed.
  const int i_end = W > 0 ? min(L, j0 + BNW - 1 + W) : L;
  const int nqt = (i_end - j0 + RQ - 1) / RQ;
  const int n_it = grp * nqt;

  i32x4 qreg[QCH], oreg[OCH];
  float sreg[3] = {0.f, 0.f, 0.f};
  auto fetch = [&](int it) {
    const int hh = kvh * grp + min(it / nqt, grp - 1);
    const int i0 = j0 + (it % nqt) * RQ;
#pragma unroll
    for (int cc = 0; cc < QCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int rr = ch / (DQK / 8), col = (ch % (DQK / 8)) * 8;
      qreg[cc] = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.q) +
                                                 ((long)(seq0 + min(i0 + rr, L - 1)) * p.Hq + hh) * DQK + col);
    }
#pragma unroll
    for (int cc = 0; cc < OCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int rr = ch / (DV / 8), col = (ch % (DV / 8)) * 8;
      oreg[cc] = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.dO) +
                                                 ((long)(seq0 + min(i0 + rr, L - 1)) * p.Hq + hh) * DV + col);
    }
    if (tid < RQ) {
      const long ri = (long)(seq0 + min(i0 + tid, L - 1)) * p.Hq + hh;
      sreg[0] = p.lse[ri];
      sreg[1] = p.delta[ri];
      sreg[2] = gated ? p.G2[ri] : 0.f;
    }
  };
  auto stash = [&](int buf, int it) {
    const int i0 = j0 + (it % nqt) * RQ;
    const i32x4 z = {0, 0, 0, 0};
#pragma unroll
    for (int cc = 0; cc < QCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int rr = ch / (DQK / 8), col = (ch % (DQK / 8)) * 8;
      *reinterpret_cast<i32x4*>(&q_lds[buf][rr * QROW + col]) = (i0 + rr < L) ? qreg[cc] : z;
    }
#pragma unroll
    for (int cc = 0; cc < OCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int rr = ch / (DV / 8), col = (ch % (DV / 8)) * 8;
      *reinterpret_cast<i32x4*>(&do_lds[buf][rr * OROW + col]) = (i0 + rr < L) ? oreg[cc] : z;
    }
    if (tid < RQ) {
      const bool ok = i0 + tid < L;
      lse_lds[buf][tid] = ok ? sreg[0] * kLog2e : 0.f;
      delta_lds[buf][tid] = ok ? sreg[1] : 0.f;
      gq_lds[buf][tid] = ok ? sreg[2] : 0.f;
    }
  };

  if constexpr (PF) {
    fetch(0);
    stash(0, 0);
    __syncthreads();
  }

  float gk[KBW], colsum[KBW];
  for (int it = 0; it < n_it; ++it) {
    const int buf = PF ? (it & 1) : 0;
    if constexpr (!PF) {
      // chunk by chunk straight into LDS: few live registers
      const int hh = kvh * grp + it / nqt;
      const int i0s = j0 + (it % nqt) * RQ;
      for (int c = tid; c < RQ * DQK / 8; c += 256) {
        const int rr = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        i32x4 val = {0, 0, 0, 0};
        if (i0s + rr < L)
          val = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.q) +
                                                ((long)(seq0 + i0s + rr) * p.Hq + hh) * DQK + col);
        *reinterpret_cast<i32x4*>(&q_lds[0][rr * QROW + col]) = val;
      }
      for (int c = tid; c < RQ * DV / 8; c += 256) {
        const int rr = c / (DV / 8), col = (c % (DV / 8)) * 8;
        i32x4 val = {0, 0, 0, 0};
        if (i0s + rr < L)
          val = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.dO) +
                                                ((long)(seq0 + i0s + rr) * p.Hq + hh) * DV + col);
        *reinterpret_cast<i32x4*>(&do_lds[0][rr * OROW + col]) = val;
      }
      if (tid < RQ) {
        const bool ok = i0s + tid < L;
        const long ri = (long)(seq0 + i0s + tid) * p.Hq + hh;
        lse_lds[0][tid] = ok ? p.lse[ri] * kLog2e : 0.f;
        delta_lds[0][tid] = ok ? p.delta[ri] : 0.f;
        gq_lds[0][tid] = (ok && gated) ? p.G2[ri] : 0.f;
      }
      __syncthreads();
    }
    const int hg = it / nqt, qt = it % nqt;
    const int h = kvh * grp + hg;
    const int i0 = j0 + qt * RQ;
    if (qt == 0) {
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const int key = jw + kb * 16 + li;
        gk[kb] = gated ? p.G2[(long)(seq0 + min(key, L - 1)) * p.Hq + h] : 0.f;
        colsum[kb] = 0.f;
      }
    }
    if constexpr (PF) fetch(it + 1);   // unconditional: indices clamped, no drain at a branch join

    // no branch around the math (see the forward kernel): masked pairs give
    // P = dS = 0; the per-element mask runs only on tiles that need it
    const bool need_mask = (i0 < jw + KW - 1) || (W > 0 && i0 + RQ - 1 - jw >= W) || (i0 + RQ > L) ||
                           (jw + KW > L);
    {
      const bf16* ql = q_lds[buf];
      const bf16* ol = do_lds[buf];
      const float* lsel = lse_lds[buf];
      const float* dell = delta_lds[buf];
      const float* gql = gq_lds[buf];
      // ---- S = Q K^T, dP = dO V^T: C lane (key li, rows rb*16+4g+i) ----
      f32x4 s[KBW][2], dp[KBW][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
          const bf16x8 a = lds_read8(ql + (rb * 16 + li) * QROW + ks * 32 + 8 * g);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) s[kb][rb] = mfma16x16x32(a, kop[kb][ks], s[kb][rb]);
        }
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          const bf16x8 a = lds_read8(ol + (rb * 16 + li) * OROW + ks * 32 + 8 * g);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) dp[kb][rb] = mfma16x16x32(a, vop[kb][ks], dp[kb][rb]);
        }
      }
      // ---- P (masked only on tiles that need it) and dS ----
      f32x4 pv[KBW][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lsel + rb * 16 + 4 * g);
        f32x4 gq4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gq4 = *reinterpret_cast<const f32x4*>(gql + rb * 16 + 4 * g);
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pv[kb][rb][i] = fast_exp2(__builtin_fmaf(s[kb][rb][i], p.scale_log2, (gq4[i] - gk[kb]) - lse4[i]));
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const int key = jw + kb * 16 + li;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = i0 + rb * 16 + 4 * g + i;
              const bool vis = key < L && row < L && key <= row && (W <= 0 || row - key < W);
              pv[kb][rb][i] = vis ? pv[kb][rb][i] : 0.f;
            }
        }
      }
      bf16x8 pop[KBW], dsop[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        f32x4 dsv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 del4 = *reinterpret_cast<const f32x4*>(dell + rb * 16 + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d = pv[kb][rb][i] * (dp[kb][rb][i] - del4[i]);
            colsum[kb] += d;
            dsv[rb][i] = d;
          }
        }
        pop[kb] = concat(to_bf16x4(pv[kb][0]), to_bf16x4(pv[kb][1]));
        dsop[kb] = concat(to_bf16x4(dsv[0]), to_bf16x4(dsv[1]));
      }
      // ---- dV^T += dO^T P, dK^T += Q^T dS (32 rows per MFMA) ----
      const int mm = li >> 2, c4 = li & 3;
      const bf16* o0 = ol + (4 * g + mm) * OROW + 4 * c4;
      const bf16* o1 = ol + (16 + 4 * g + mm) * OROW + 4 * c4;
      // (compiler barriers every few column blocks keep the scheduler from
      //  hoisting every transposed read at once and running out of registers)
#pragma unroll
      for (int db = 0; db < DBV; ++db) {
        const bf16x8 a = concat(lds_read_tr16(o0 + db * 16), lds_read_tr16(o1 + db * 16));
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) dv_acc[kb][db] = mfma16x16x32(a, pop[kb], dv_acc[kb][db]);
        if ((db & 3) == 3) asm volatile("" ::: "memory");
      }
      const bf16* q0 = ql + (4 * g + mm) * QROW + 4 * c4;
      const bf16* q1 = ql + (16 + 4 * g + mm) * QROW + 4 * c4;
#pragma unroll
      for (int db = 0; db < DBQ; ++db) {
        const bf16x8 a = concat(lds_read_tr16(q0 + db * 16), lds_read_tr16(q1 + db * 16));
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) dk_acc[kb][db] = mfma16x16x32(a, dsop[kb], dk_acc[kb][db]);
        if ((db & 3) == 3) asm volatile("" ::: "memory");
      }
    }
    if (gated && qt == nqt - 1) {
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const float cs = xgroup_sum(colsum[kb]);
        const int key = jw + kb * 16 + li;
        if (g == 0 && key < L) p.dGcol[(long)(seq0 + key) * p.Hq + h] = cs;
      }
    }
    if constexpr (PF) {
      if (it + 1 < n_it) stash(buf ^ 1, it + 1);
    }
    __syncthreads();
  }

#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int key = jw + kb * 16 + li;
    if (key >= L) continue;
    bf16* dkp = reinterpret_cast<bf16*>(p.dk) + ((long)(seq0 + key) * p.Hkv + kvh) * DQK + 4 * g;
    bf16* dvp = reinterpret_cast<bf16*>(p.dv) + ((long)(seq0 + key) * p.Hkv + kvh) * DV + 4 * g;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) *reinterpret_cast<bf16x4*>(dkp + db * 16) = to_bf16x4(dk_acc[kb][db] * p.scale);
#pragma unroll
    for (int db = 0; db < DBV; ++db) *reinterpret_cast<bf16x4*>(dvp + db * 16) = to_bf16x4(dv_acc[kb][db]);
  }
}

// ---------------------------------------------------------------------------
template <int DQK, int DV, int RW, int BN, bool GATED>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = 4 * RW;
  constexpr int RBW = RW / 16;
  constexpr int KB = BN / 16;
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int DBQ = DQK / 16;
  constexpr int KROW = DQK + 8, VROW = DV + 16;
  constexpr int KCH = BN * DQK / 8 / 256, VCH = BN * DV / 8 / 256;
  static_assert(KB % 2 == 0, "dQ consumes keys in pairs of 16-key blocks");
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2][BN * VROW];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][BN];

  const int h = xcd_remap(blockIdx.x, p.Hq), n = blockIdx.y;
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
  const int r0 = i0 + wave * RW;
  const int r_last = min(r0 + RW, L) - 1;

  bf16x8 qop[RBW][KSQ], doop[RBW][KSV];
  float lse2[RBW], dlt[RBW], gq[RBW], rowsum[RBW], pdp[RBW];
  f32x4 dq_acc[RBW][DBQ];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = r0 + rb * 16 + li;
    const bool ok = row < L;
    const long ri = (long)(seq0 + min(row, L - 1)) * p.Hq + h;
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + ri * DQK + 8 * g;
    const bf16* dp = reinterpret_cast<const bf16*>(p.dO) + ri * DV + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qop[rb][ks] = ok ? *reinterpret_cast<const bf16x8*>(qp + 32 * ks) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) doop[rb][ks] = ok ? *reinterpret_cast<const bf16x8*>(dp + 32 * ks) : bf16x8{};
    lse2[rb] = ok ? p.lse[ri] * kLog2e : 0.f;
    dlt[rb] = ok ? p.delta[ri] : 0.f;
    gq[rb] = (ok && gated) ? p.G2[ri] : 0.f;
    rowsum[rb] = 0.f;
    pdp[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) dq_acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BM);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long)seq0 * p.Hkv + kvh) * DQK;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long)seq0 * p.Hkv + kvh) * DV;
  const long kstride = (long)p.Hkv * DQK, vstride = (long)p.Hkv * DV;

  i32x4 kreg[KCH], vreg[VCH];
  float gkreg = 0.f;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int cc = 0; cc < KCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DQK / 8), col = (ch % (DQK / 8)) * 8;
      kreg[cc] = *reinterpret_cast<const i32x4*>(kbase + (long)min(j0 + kr, L - 1) * kstride + col);
    }
#pragma unroll
    for (int cc = 0; cc < VCH; ++cc) {
      const int ch = tid + 256 * cc;
      const int kr = ch / (DV / 8), col = (ch % (DV / 8)) * 8;
      vreg[cc] = *reinterpret_cast<const i32x4*>(vbase + (long)min(j0 + kr, L - 1) * vstride + col);
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
    fetch(j0 + BN);   // unconditional: clamped addresses, no drain at a branch join

    // no branch around the math (see the forward kernel): wholly masked
    // tiles contribute zeros; rows past the end are masked too, their lse
    // is not defined
    {
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + RW - 1);
      const bf16* kl = k_lds[buf];
      const bf16* vl = v_lds[buf];
      f32x4 s[KB][RBW], dp[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
          const bf16x8 a = lds_read8(kl + (kb * 16 + li) * KROW + ks * 32 + 8 * g);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) s[kb][rb] = mfma16x16x32(a, qop[rb][ks], s[kb][rb]);
        }
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          const bf16x8 a = lds_read8(vl + (kb * 16 + li) * VROW + ks * 32 + 8 * g);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) dp[kb][rb] = mfma16x16x32(a, doop[rb][ks], dp[kb][rb]);
        }
      }
      // ---- P (masked only on tiles that need it), dS, row sums ----
      f32x4 pv[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 gk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(&gk_lds[buf][kb * 16 + 4 * g]);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const float base = gq[rb] - lse2[rb];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[kb][rb][i] = fast_exp2(__builtin_fmaf(s[kb][rb][i], c, base - gk[i]));
        }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            const int row = r0 + rb * 16 + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = j0 + kb * 16 + 4 * g + i;
              const bool vis = key <= row && key < L && row < L && (W <= 0 || row - key < W);
              pv[kb][rb][i] = vis ? pv[kb][rb][i] : 0.f;
            }
          }
      }
      bf16x4 dsb[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          f32x4 dsv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = pv[kb][rb][i];
            const float d = pr * (dp[kb][rb][i] - dlt[rb]);
            pdp[rb] += pr * dp[kb][rb][i];
            rowsum[rb] += d;
            dsv[i] = d;
          }
          dsb[kb][rb] = to_bf16x4(dsv);
        }
      // ---- dQ^T += K^T dS^T, 32 keys per MFMA ----
#pragma unroll
      for (int kp = 0; kp < KB / 2; ++kp) {
        const int mm = li >> 2, c4 = li & 3;
        const bf16* k0 = kl + (kp * 32 + 4 * g + mm) * KROW + 4 * c4;
        const bf16* k1 = kl + (kp * 32 + 16 + 4 * g + mm) * KROW + 4 * c4;
#pragma unroll
        for (int db = 0; db < DBQ; ++db) {
          const bf16x8 a = concat(lds_read_tr16(k0 + db * 16), lds_read_tr16(k1 + db * 16));
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            dq_acc[rb][db] = mfma16x16x32(a, concat(dsb[2 * kp][rb], dsb[2 * kp + 1][rb]), dq_acc[rb][db]);
        }
      }
    }
    if (more) stash(buf ^ 1, j0 + BN);
    __syncthreads();
  }

  const float sink2 = p.sink ? p.sink[h] * kLog2e : 0.f;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = r0 + rb * 16 + li;
    const float rs = xgroup_sum(rowsum[rb]);
    const float sp = xgroup_sum(pdp[rb]);
    if (row >= L) continue;
    const long ri = (long)(seq0 + row) * p.Hq + h;
    bf16* dqp = reinterpret_cast<bf16*>(p.dq) + ri * DQK + 4 * g;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) *reinterpret_cast<bf16x4*>(dqp + db * 16) = to_bf16x4(dq_acc[rb][db] * p.scale);
    if (g == 0) {
      if (gated) p.dGrow[ri] = rs;
      if (p.sink) p.sink_rows[ri] = fast_exp2(sink2 - lse2[rb]) * sp;
    }
  }
}

// dsink[h] = -sum over all tokens of sink_rows[t, h] (fixed order).
__global__ __launch_bounds__(256) void sink_reduce_kernel(const float* __restrict__ rows, float* __restrict__ dsink,
                                                          int T, int Hq) {
  const int h = blockIdx.x;
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) s += rows[(long)t * Hq + h];
  __shared__ float part[256];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsink[h] = -part[0];
}

template <int DQK, int DV, int KW, int RW, int BN>
hipError_t launch_bwd_two_pass_t(const BwdParams& p, hipStream_t st) {
  const int ktiles = (p.max_seqlen + 4 * KW - 1) / (4 * KW);
  const dim3 gk(p.Hkv, p.num_seqs, ktiles);
  if (p.G2) bwd_dkdv_kernel<DQK, DV, KW, (DV <= 256), true><<<gk, 256, 0, st>>>(p);
  else bwd_dkdv_kernel<DQK, DV, KW, (DV <= 256), false><<<gk, 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int qtiles = (p.max_seqlen + 4 * RW - 1) / (4 * RW);
  const dim3 gq(p.Hq, p.num_seqs, qtiles);
  if (p.G2) bwd_dq_kernel<DQK, DV, RW, BN, true><<<gq, 256, 0, st>>>(p);
  else bwd_dq_kernel<DQK, DV, RW, BN, false><<<gq, 256, 0, st>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.sink) {
    sink_reduce_kernel<<<dim3(p.Hq), 256, 0, st>>>(p.sink_rows, p.dsink_acc, p.T, p.Hq);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd_two_pass(const BwdParams& p, int dqk, int dv, hipStream_t st) {
  if (dqk == 64 && dv == 64) return launch_bwd_two_pass_t<64, 64, BWD_KW_SMALL, BWD_RW_SMALL, 64>(p, st);
  if (dqk == 128 && dv == 128) return launch_bwd_two_pass_t<128, 128, BWD_KW_SMALL, BWD_RW_SMALL, 64>(p, st);
  if (dqk == 256 && dv == 256) return launch_bwd_two_pass_t<256, 256, 16, 16, 32>(p, st);
  if (dqk == 256 && dv == 512) return launch_bwd_two_pass_t<256, 512, 16, 16, 32>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
