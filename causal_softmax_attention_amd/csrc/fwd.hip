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
#ifndef FWD_NST_SMALL
#define FWD_NST_SMALL 2
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

template <int DQK, int DV, int RW, int BN, int NST, bool GATED>
__global__ __launch_bounds__(256) void fwd_kernel(FwdParams p) {
  constexpr int BM = 4 * RW;
  constexpr int RBW = RW / 16;       // 16-row blocks per wave
  constexpr int KB = BN / 16;        // 16-key blocks per tile
  constexpr int KS = DQK / 32;       // k-steps over d_qk
  constexpr int DB = DV / 16;        // 16-wide output column blocks
  constexpr int KRB = DQK * 2, VRB = DV * 2;   // bytes per K / V row
  static_assert(KB % 2 == 0, "PV consumes keys in pairs of 16-key blocks");
  static_assert(NST >= 2 && BN <= 64, "ring of at least two stages; gate copy is one lane per key");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[NST][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[NST][BN * VRB];
  __shared__ __attribute__((aligned(16))) float gk_lds[NST][4][64];   // one copy per wave

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
      gq[rb] = GATED ? p.G2[(long)(seq0 + row) * p.Hq + h] : 0.f;
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

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + ((long)seq0 * p.Hkv + kvh) * VRB;
  const long kstride = (long)p.Hkv * KRB, vstride = (long)p.Hkv * VRB;

  // K/V tiles (and each wave's copy of the key-side gate terms) go global ->
  // LDS directly, NST-1 tiles ahead of the math, into a ring of NST stages.
  // Every wave issues the same number of loads per tile, so the wait for
  // the oldest tile is an exact vmcnt.
  constexpr int LOADS_PER_TILE = (BN * KRB + BN * VRB) / 4096 + (GATED ? 1 : 0);
  const int G2_tok_stride = p.Hq;
  TileDma<KRB, BN> kdma;
  TileDma<VRB, BN> vdma;
  kdma.init(kstride, wave, lane);
  vdma.init(vstride, wave, lane);
  auto fetch = [&](int st, int j0) {
    kdma.issue(kbase, kstride, j0, L, k_lds[st], wave);
    vdma.issue(vbase, vstride, j0, L, v_lds[st], wave);
    if constexpr (GATED) {
      const float* src = p.G2 + (long)(seq0 + min(j0 + lane, L - 1)) * G2_tok_stride + h;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void LDS_AS*)(&gk_lds[st][wave][0]), 4, 0, 0);
    }
  };
  auto wait_tiles_in_flight = [&](int n) {   // oldest tile landed when <= n tiles remain in flight
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS_PER_TILE) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LOADS_PER_TILE) : "memory");
  };

  // prologue: tiles t_begin .. t_begin+NST-2
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (t_begin + s < t_end) fetch(s, (t_begin + s) * BN);

  for (int t = t_begin; t < t_end; ++t) {
    const int j0 = t * BN;
    const int st = (t - t_begin) % NST;
    // tiles issued after this one and still possibly in flight
    wait_tiles_in_flight(min(NST - 2, t_end - 1 - t));
    __syncthreads();
    if (t + NST - 1 < t_end) fetch((t - t_begin + NST - 1) % NST, (t + NST - 1) * BN);

    // No branch around the math: a tile that is wholly masked for this
    // wave's rows goes through the masked path and contributes zeros.  (A
    // branch here makes the compiler shuttle every accumulator between
    // AGPRs and VGPRs on each iteration.)
    {
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + RW - 1);
      const uint8_t* kl = k_lds[st];
      const uint8_t* vl = v_lds[st];
      const float* gkl = gk_lds[st][wave];
      // ---- S^T = K Q^T ----
      f32x4 sc[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + tile_off<KRB>(kb * 16 + li, 64 * ks + 16 * g));
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = mfma16x16x32(a, qop[rb][ks], sc[kb][rb]);
        }
      }
      // ---- y = s*c - gk (base 2, without the row's gate term) ----
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 gk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(gkl + kb * 16 + 4 * g);
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
      const int mm = li >> 2, c4 = li & 3;
#pragma unroll
      for (int kp = 0; kp < KB / 2; ++kp) {
        const int vr0 = kp * 32 + 4 * g + mm, vr1 = vr0 + 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(vl + tile_off<VRB>(vr0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(vl + tile_off<VRB>(vr1, b))));
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            oacc[rb][db] = mfma16x16x32(a, concat(pb[2 * kp][rb], pb[2 * kp + 1][rb]), oacc[rb][db]);
        }
      }
    }
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

template <int DQK, int DV, int RW, int BN, int NST>
static hipError_t launch_cfg(const FwdParams& p, hipStream_t st) {
  constexpr int BM = 4 * RW;
  const int tiles = (p.max_seqlen + BM - 1) / BM;
  dim3 grid(p.Hq, p.num_seqs, tiles), block(256);
  if (p.G2 != nullptr)
    fwd_kernel<DQK, DV, RW, BN, NST, true><<<grid, block, 0, st>>>(p);
  else
    fwd_kernel<DQK, DV, RW, BN, NST, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, hipStream_t st) {
  if (p.num_seqs == 0 || p.T == 0 || p.max_seqlen == 0) return hipSuccess;
  if (dqk == 64 && dv == 64) return launch_cfg<64, 64, FWD_RW_SMALL, FWD_BN_SMALL, FWD_NST_SMALL>(p, st);
  if (dqk == 128 && dv == 128) return launch_cfg<128, 128, FWD_RW_SMALL, FWD_BN_SMALL, FWD_NST_SMALL>(p, st);
  if (dqk == 256 && dv == 256) return launch_cfg<256, 256, 16, 32, 2>(p, st);
  if (dqk == 256 && dv == 512) return launch_cfg<256, 512, 16, 32, 2>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
