// Software-pipelined packed variable-length causal attention forward for
// gfx950, head dims 64 and 128.
//
// Method (fla issue #1322, Description): causal softmax attention over
// packed sequences with GQA/MQA, a logarithmic gate bias G_i - G_j (G the
// per-sequence inclusive cumsum of the log gates), a sliding window and a
// per-head sink logit that adds e^sink to the softmax denominator without a
// value.  Scores accumulate in fp32 from bf16 operands; probabilities enter
// PV as bf16 (round to nearest even); O is rounded to bf16 at the end and
// lse is kept in fp32.
//
// gfx950 mapping
//  * One workgroup of four wavefronts per (HPW query heads of one KV head,
//    query tile, sequence); wave w takes head w % HPW and 32 query rows
//    (4 / HPW row groups).  With HPW = 4 (GQA 4 and wider) the four heads of
//    a KV group share each K/V tile in LDS, and every wave sees the same key
//    range.  The grid is sequence-major (all tiles of a sequence are
//    dispatched together, longest first), and the workgroups of one KV head
//    run on one XCD: the window of K/V that a sequence's tiles share stays
//    in that XCD's L2 (measured 348 -> 278 us on the 8-sequence window-1024
//    workload against the head-major order).
//  * v_mfma_f32_32x32x16_bf16 for both products: S^T = K Q^T with Q in
//    registers, so each lane owns one query row (its max and sum need one
//    lane swap), and O^T += V^T P^T with V^T from ds_read_b64_tr_b16, so P
//    goes from the score registers into the PV MFMA without a shuffle.  The
//    32x32 shape halves the MFMA count of 16x16x32 for the same work and
//    hides more VALU work per MFMA (measured on gfx950: four VALU ops after
//    a 32x32x16 MFMA add ~4 cycles to its 32, two after a 16x16x32 add ~6 to
//    its 16).
//  * K and V tiles of 64 keys reach LDS by direct global->LDS copies into
//    two-stage rings; each tile has its own swizzle, conflict-free for its
//    read pattern (K: MFMA A-operand rows, V: transposed reads).
//  * The tile loop is software pipelined inside each wave: iteration t
//    computes S(t) = K(t) Q^T while the exponentials, row sums and bf16
//    conversion of tile t-1 run between its MFMAs (block A), then
//    accumulates P(t-1) V(t-1) while the gate bias and row max of S(t) run
//    between those MFMAs (block B).  Both blocks are written slot by slot
//    (one MFMA, its share of LDS reads and VALU work) with a scheduling
//    fence per slot, so the compiler keeps that interleave.
//  * Online softmax in base 2 with a lazy rescale: scores are scaled by
//    softmax_scale * log2(e), the gate prefix is stored pre-multiplied by
//    log2(e), the running max starts at the sink logit with l = 1, and it
//    is raised only when a tile's max passes it by more than kRescaleSlack.
//    Masking (diagonal, window edge, sequence end) runs only on the tiles
//    that cross one of them, on the raw scores (softmax_scale > 0).
#pragma once
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace attn {

// Maps a block index so that consecutive logical indices share one XCD
// (blocks are dispatched round-robin over the 8 XCDs, each with its own L2).
__device__ __forceinline__ int xcd_group(int x, int n) {
  if (n % 8 != 0) return x;
  return (x % 8) * (n / 8) + x / 8;
}

// Swizzles of the K and V tiles (16-byte chunk c of row r is stored at
// chunk position c ^ swz(r)).  K is read as MFMA A-operand rows: 32 lanes
// read the same chunk of 32 consecutive rows, served over 512 bytes of
// banks, so the rows that share a bank line (every 512 / RB-th row) must
// land on different chunks.  V is read transposed: 32 lanes read 64 bytes of
// 4 consecutive rows, served over 256 bytes of banks, so those 4 rows must
// land on different 64-byte segments.
template <int RB>
__device__ __forceinline__ int swz_k32(int r) {
  return RB == 256 ? ((r >> 1) & 15) : ((r >> 2) & 7);
}
template <int RB>
__device__ __forceinline__ int swz_v32(int r) {
  return RB == 256 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Lane layout of v_mfma_f32_32x32x16_bf16 (checked on gfx950 with an
// in-bounds probe; l = lane, h = l / 32):
//   A[m][k]: m = l % 32, k = 8 h + e (e = 0..7)
//   B[k][n]: n = l % 32, k = 8 h + e
//   C[m][n]: n = l % 32, m = 8 (i / 4) + 4 h + i % 4 (i = 0..15)
// S^T = K Q^T: each lane owns one query row (l % 32) and 16 keys of every
// 32-key block; lanes l and l ^ 32 share the row.  P^T for PV k-step s
// (16 keys) is C registers 8 (s % 2) .. 8 (s % 2) + 7 of key block s / 2,
// i.e. keys 16 s + 8 (e / 4) + 4 h + e % 4 for element e; V^T is read with
// the same key order (two transposed reads of 4 keys each).
template <int DQK, int DV, bool GATED, int HPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_pipe_kernel(FwdParams p) {
  constexpr int RW = 32;                 // query rows per wave
  constexpr int WPH = 4 / HPW;           // waves (row groups) per head
  constexpr int BM = RW * WPH;           // query rows per workgroup
  constexpr int BN = 64, KB = BN / 32;   // keys per tile, 32-key blocks per tile
  constexpr int KS = DQK / 16;           // QK k-steps
  constexpr int DB = DV / 32;            // 32-wide output column blocks
  constexpr int PS = BN / 16;            // PV k-steps
  constexpr int KRB = DQK * 2, VRB = DV * 2;   // bytes per K / V row
  constexpr int KPW = BN * KRB / 4096, VPW = BN * VRB / 4096;   // 1 KB copies per wave per tile
  static_assert(KPW * 4096 == BN * KRB && VPW * 4096 == BN * VRB, "tile must split into 4 x k 1 KB blocks");
  static_assert((KRB == 128 || KRB == 256) && (VRB == 128 || VRB == 256), "head dims 64 or 128");
  static_assert(HPW == 1 || HPW == 2 || HPW == 4, "heads per workgroup");
  constexpr int NQK = KB * KS;           // QK MFMAs per tile
  constexpr int NPV = PS * DB;           // PV MFMAs per tile
  constexpr int NE = KB * 16;            // score elements per lane per tile
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][BN * VRB];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][4][BN];   // per wave: its head's key gate terms

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;   // row within the wave, lane half
  const int hx = xcd_group(blockIdx.x, p.Hq / HPW);
  const int h = hx * HPW + wave % HPW;
  const int kvh = h / (p.Hq / p.Hkv);
  const int n = blockIdx.z;
  const int tile = gridDim.y - 1 - blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int i0 = tile * BM;
  if (i0 >= L) return;
  const int W = p.window;
  const float c = p.scale_log2;

  const int r0 = i0 + (wave / HPW) * RW;   // first row of this wave
  const int r_last = min(r0 + RW, L) - 1;  // last real row (may be < r0)
  const int row = r0 + lr;                 // this lane's query row

  // ---- Q operand (B of S^T = K Q^T) and per-row state; the running max is
  //      kept without the row's own gate term gq ----
  bf16x8 qop[KS];
  float gq = 0.f;
  if (row < L) {
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + ((long)(seq0 + row) * p.Hq + h) * DQK + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
    if constexpr (GATED) gq = p.G2[(long)h * p.T + seq0 + row];
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = bf16x8{};
  }
  const float sink2 = p.sink ? p.sink[h] * kLog2e : kNegBig;
  float m_run = p.sink ? sink2 - gq : kNegBig;
  float l_run = p.sink ? 1.f : 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // ---- key range of the workgroup, and of this wave ----
  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BM);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;
  int tw_lo = t_begin, tw_hi = t_begin;
  if (r_last >= r0) {
    tw_lo = (W > 0 && r0 - W + 1 > 0) ? max(t_begin, (r0 - W + 1) / BN) : t_begin;
    tw_hi = min(t_end, r_last / BN + 1);
    tw_lo = min(tw_lo, tw_hi);
  }

  // ---- tile copies.  Wave w copies the 1 KB blocks w, w+4, ... of each
  // tile; lane l fills bytes 16 l .. 16 l + 15 of its block: tile row
  // (1024 j + 16 l) / RB at chunk position p, which holds logical chunk
  // p ^ swz(row).  Only the last tile of a sequence clamps rows past the end
  // to the last row (in range and finite; those keys are masked). ----
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + ((long)seq0 * p.Hkv + kvh) * VRB;
  const int kstride = p.Hkv * KRB, vstride = p.Hkv * VRB;
  int koff[KPW], voff[VPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    const int r = o / KRB;
    koff[j] = r * kstride + ((((o % KRB) >> 4) ^ swz_k32<KRB>(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    const int r = o / VRB;
    voff[j] = r * vstride + ((((o % VRB) >> 4) ^ swz_v32<VRB>(r)) << 4);
  }
  const float* g2base = GATED ? p.G2 + (long)h * p.T + seq0 : nullptr;
  auto fetch_k = [&](int t) {
    const int j0 = t * BN, st = (t - t_begin) & 1;
    const uint8_t* kb = kbase + (long)j0 * kstride;
    const uint32_t kl = lds_addr(k_lds[st]);
    if (j0 + BN > L) {   // uniform: only the last tile of a sequence clamps
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int r = ((wave + 4 * j) * 1024 + lane * 16) / KRB;
        const int over = max(0, j0 + r - (L - 1));
        dma16(kb, (uint32_t)(koff[j] - over * kstride), kl + (wave + 4 * j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPW; ++j) dma16(kb, (uint32_t)koff[j], kl + (wave + 4 * j) * 1024);
    }
    if constexpr (GATED) dma4(g2base, (uint32_t)(min(j0 + lane, L - 1) * 4), lds_addr(&gk_lds[st][wave][0]));
  };
  auto fetch_v = [&](int t) {
    const int j0 = t * BN, st = (t - t_begin) & 1;
    const uint8_t* vb = vbase + (long)j0 * vstride;
    const uint32_t vl = lds_addr(v_lds[st]);
    if (j0 + BN > L) {
#pragma unroll
      for (int j = 0; j < VPW; ++j) {
        const int r = ((wave + 4 * j) * 1024 + lane * 16) / VRB;
        const int over = max(0, j0 + r - (L - 1));
        dma16(vb, (uint32_t)(voff[j] - over * vstride), vl + (wave + 4 * j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPW; ++j) dma16(vb, (uint32_t)voff[j], vl + (wave + 4 * j) * 1024);
    }
  };

  // ---- per-lane LDS operand addresses.  K fragment (key block kb, k-step
  // ks): row 32 kb + lr, logical chunk 2 ks + hh, i.e. the ks = 0 address
  // XOR 32 ks (row offsets and stage bases have no bits in the chunk field).
  // V^T fragment (PV k-step s, column block db, read j2): row 16 s + 8 j2 +
  // 4 hh + j (j = (l % 16) / 4), logical chunk 4 db + 2 half + cc / 2 (half =
  // (l / 16) % 2, cc = l % 4), i.e. the db = 0 address XOR 64 db. ----
  const uint32_t k_lane0 = (uint32_t)(lr * KRB + ((hh ^ swz_k32<KRB>(lr)) << 4));
  const int vj = (lane & 15) >> 2, vc = lane & 3, vhalf = (lane >> 4) & 1;
  const int vrow = 4 * hh + vj;
  const uint32_t v_lane0 =
      (uint32_t)(vrow * VRB + (((2 * vhalf + (vc >> 1)) ^ swz_v32<VRB>(vrow)) << 4) + 8 * (vc & 1));
  auto k_addr = [&](int t, int ks) {
    uint32_t a = (lds_addr(k_lds[(t - t_begin) & 1]) + k_lane0) ^ (uint32_t)(32 * ks);
    asm volatile("" : "+v"(a));   // keeps the constant tile offsets in the reads' offset fields
    return (const LDS_AS uint8_t*)a;
  };
  auto v_addr = [&](int t, int db) {
    uint32_t a = (lds_addr(v_lds[(t - t_begin) & 1]) + v_lane0) ^ (uint32_t)(64 * db);
    asm volatile("" : "+v"(a));
    return (const LDS_AS uint8_t*)a;
  };

  // ---- iteration t: wait for K(t) (and its gate terms) and V(t-1), release
  // them to the workgroup, put K(t+1) and V(t) in flight.  Every wave takes
  // part in every iteration t_begin .. t_end. ----
  fetch_k(t_begin);
  auto sync = [&](int t) {
    wait_vm<0>();
    lds_barrier();
    if (t + 1 < t_end) fetch_k(t + 1);
    if (t < t_end) fetch_v(t);
  };

  // mask of tile t on the raw scores (c > 0, so -inf stays -inf after
  // scaling); the empty asm keeps it a branch taken only on the tiles that
  // cross the diagonal, the window edge or the end
  auto mask = [&](int t, f32x16 (&s)[KB]) {
    asm volatile("" ::: "memory");
    const int j0 = t * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = j0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool vis = key <= row && key < L && (W <= 0 || row - key < W);
        s[kb][i] = vis ? s[kb][i] : -INFINITY;
      }
  };
  auto need_mask = [&](int t) {
    const int j0 = t * BN;
    return (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) || (r_last < r0 + RW - 1);
  };
  float mx = -INFINITY;   // row max of the newest tile
  // lazy rescale against the new row max
  auto rescale = [&]() {
    if (__builtin_expect(__any(mx > m_run + kRescaleSlack), 0)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
  };

  // Exponent work (block A) on y (the previous tile): element e = (kb, i)
  // with e = 16 kb + i; every 8 elements form the bf16 P operand of one PV
  // k-step and add their sum to the row sum.
  bf16x8 pb[PS];
  float rsum = 0.f;
  auto exp_elem = [&](f32x16 (&y)[KB], int e) { y[e / 16][e % 16] = fast_exp2(y[e / 16][e % 16] - m_run); };
  auto exp_group = [&](f32x16 (&y)[KB], int gi) {   // after its 8 exps
    const int kb = gi / 2, o = 8 * (gi % 2);
    const float pt = ((y[kb][o] + y[kb][o + 1]) + (y[kb][o + 2] + y[kb][o + 3])) +
                     ((y[kb][o + 4] + y[kb][o + 5]) + (y[kb][o + 6] + y[kb][o + 7]));
    rsum = gi == 0 ? pt : rsum + pt;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)y[kb][o + e];
    pb[gi] = v;
  };
  auto exp_row = [&]() {   // after all groups
    const unsigned u = __float_as_uint(rsum);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_run += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // fp32 row sum: lse feeds the backward
  };
  auto exp_slot = [&](f32x16 (&y)[KB], int j, auto ns) {
    constexpr int per = NE / decltype(ns)::value;
#pragma unroll
    for (int q = 0; q < per; ++q) exp_elem(y, j * per + q);
    if (j > 0) {
#pragma unroll
      for (int e = (j - 1) * per; e < j * per; ++e)
        if (e % 8 == 7) exp_group(y, e / 8);
    }
  };
  auto exp_tail = [&](f32x16 (&y)[KB], auto ns) {
    constexpr int NS = decltype(ns)::value, per = NE / NS;
#pragma unroll
    for (int e = (NS - 1) * per; e < NE; ++e)
      if (e % 8 == 7) exp_group(y, e / 8);
    exp_row();
  };

  // Bias work (block B) on the fresh scores s: y = s c - gk (gated) or s c,
  // in place, and the running row max.
  f32x4 gk4[2];
  const float* gkl = nullptr;
  float mrow = -INFINITY;
  auto gk_read = [&](int gi) {   // gate terms of keys 32 (gi / 4) + 8 (gi % 4) + 4 hh .. + 3
    if constexpr (GATED) gk4[gi & 1] = *reinterpret_cast<const f32x4*>(gkl + 8 * gi + 4 * hh);
  };
  auto bias_elem = [&](f32x16 (&s)[KB], int e) {
    const int kb = e / 16, i = e % 16, gi = e / 4;
    if constexpr (GATED) {
      if (i % 4 == 0 && gi + 1 < NE / 4) gk_read(gi + 1);
      s[kb][i] = __builtin_fmaf(s[kb][i], c, -gk4[gi & 1][i % 4]);
    } else {
      s[kb][i] = s[kb][i] * c;
    }
  };
  auto bias_slot = [&](f32x16 (&s)[KB], int j, auto ns) {
    constexpr int per = NE / decltype(ns)::value;
#pragma unroll
    for (int q = 0; q < per; ++q) bias_elem(s, j * per + q);
    if (j > 0) {
      // max of the elements biased in the previous slot
      const int e0 = (j - 1) * per;
      if constexpr (per == 2) mrow = fmaxf(mrow, fmaxf(s[e0 / 16][e0 % 16], s[(e0 + 1) / 16][(e0 + 1) % 16]));
      else {
#pragma unroll
        for (int e = 0; e < per; ++e) mrow = fmaxf(mrow, s[(e0 + e) / 16][(e0 + e) % 16]);
      }
    }
  };
  auto bias_tail = [&](f32x16 (&s)[KB], auto ns) {
    constexpr int NS = decltype(ns)::value, per = NE / NS;
#pragma unroll
    for (int e = (NS - 1) * per; e < NE; ++e) mrow = fmaxf(mrow, s[e / 16][e % 16]);
    const unsigned u = __float_as_uint(mrow);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    mx = max_nq(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  auto bias_begin = [&](int t) {
    if constexpr (GATED) {
      gkl = gk_lds[(t - t_begin) & 1][wave];
      gk_read(0);
    }
    mrow = -INFINITY;
  };

  // Block A: S(t) = K(t) Q^T into snew, slot by slot, with the exponent work
  // of yold between the MFMAs; K fragments are read FA_LEAD MFMAs ahead.
  constexpr int FA_LEAD = 3, FA_NB = FA_LEAD + 1;
  auto block_a = [&](int t, f32x16 (&snew)[KB], f32x16 (&yold)[KB], bool ex) {
    const LDS_AS uint8_t* ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = k_addr(t, ks);
    bf16x8 kf[FA_NB];
    auto kread = [&](int f) {   // fragment f = (kb = f / KS, ks = f % KS)
      kf[f % FA_NB] = *reinterpret_cast<const LDS_AS bf16x8*>(ka[f % KS] + (f / KS) * 32 * KRB);
    };
#pragma unroll
    for (int f = 0; f < FA_LEAD && f < NQK; ++f) kread(f);
#pragma unroll
    for (int sl = 0; sl < NQK; ++sl) {
      const int kb = sl / KS, ks = sl % KS;
      if (sl + FA_LEAD < NQK) kread(sl + FA_LEAD);
      snew[kb] = mfma32x32x16(kf[sl % FA_NB], qop[ks], ks == 0 ? f32x16{} : snew[kb]);
      if (ex) exp_slot(yold, sl, std::integral_constant<int, NQK>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ex) exp_tail(yold, std::integral_constant<int, NQK>{});
  };
  // Block B: O^T += V^T(t-1) P^T slot by slot, with the bias and max work of
  // s between the MFMAs; V^T fragments (two transposed reads) are read
  // FB_LEAD MFMAs ahead.
  constexpr int FB_LEAD = 2, FB_NB = FB_LEAD + 1;
  auto block_b = [&](int t, f32x16 (&s)[KB], bool pvon) {
    bias_begin(t);
    if (!pvon) {
#pragma unroll
      for (int j = 0; j < 16; ++j) bias_slot(s, j, std::integral_constant<int, 16>{});
      bias_tail(s, std::integral_constant<int, 16>{});
      return;
    }
    const LDS_AS uint8_t* va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = v_addr(t - 1, db);
    bf16x8 vf[FB_NB];
    auto vread = [&](int f) {   // fragment f = (k-step s = f / DB, column block db = f % DB)
      const int ps = f / DB, db = f % DB;
      vf[f % FB_NB] = concat(lds_tr16(va[db] + 16 * ps * VRB), lds_tr16(va[db] + (16 * ps + 8) * VRB));
    };
#pragma unroll
    for (int f = 0; f < FB_LEAD && f < NPV; ++f) vread(f);
#pragma unroll
    for (int sl = 0; sl < NPV; ++sl) {
      const int ps = sl / DB, db = sl % DB;
      if (sl + FB_LEAD < NPV) vread(sl + FB_LEAD);
      oacc[db] = mfma32x32x16(vf[sl % FB_NB], pb[ps], oacc[db]);
      bias_slot(s, sl, std::integral_constant<int, NPV>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    bias_tail(s, std::integral_constant<int, NPV>{});
  };
  // plain PV (epilogue)
  auto pv_only = [&](int t) {
    const LDS_AS uint8_t* va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = v_addr(t - 1, db);
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a = concat(lds_tr16(va[db] + 16 * ps * VRB), lds_tr16(va[db] + (16 * ps + 8) * VRB));
        oacc[db] = mfma32x32x16(a, pb[ps], oacc[db]);
      }
  };

  f32x16 sA[KB], sB[KB];
  // prologue: S(tw_lo) -> y, max, rescale
  auto first = [&](int t, f32x16 (&s)[KB]) {
    sync(t);
    block_a(t, s, sB, false);
    if (need_mask(t)) mask(t, s);
    block_b(t, s, false);
    rescale();
  };
  // steady state: S(t) into snew while P(t-1) is formed from yold, then
  // PV(t-1) while y(t) and its max are formed
  auto full = [&](int t, f32x16 (&snew)[KB], f32x16 (&yold)[KB]) {
    sync(t);
    block_a(t, snew, yold, true);
    if (need_mask(t)) mask(t, snew);
    block_b(t, snew, true);
    rescale();
  };
  // epilogue: P(t-1) and PV(t-1)
  auto last = [&](int t, f32x16 (&yold)[KB]) {
    sync(t);
#pragma unroll
    for (int j = 0; j < 16; ++j) exp_slot(yold, j, std::integral_constant<int, 16>{});
    exp_tail(yold, std::integral_constant<int, 16>{});
    pv_only(t);
  };

  int t = t_begin;
  for (; t < tw_lo; ++t) sync(t);
  if (tw_lo < tw_hi) {
    first(t, sA);
    ++t;
    for (; t + 1 < tw_hi; t += 2) {
      full(t, sB, sA);
      full(t + 1, sA, sB);
    }
    if (t < tw_hi) {
      full(t, sB, sA);
      last(t + 1, sB);
    } else {
      last(t, sA);
    }
    t = tw_hi + 1;
  }
  for (; t <= t_end; ++t) sync(t);

  // ---- finalize: O = acc / l, lse = ln 2 * (m + gq + log2 l) ----
  if (row < L) {
    const float inv = 1.0f / l_run;
    bf16* op = reinterpret_cast<bf16*>(p.o) + ((long)(seq0 + row) * p.Hq + h) * DV + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = f32x4{oacc[db][4 * q], oacc[db][4 * q + 1], oacc[db][4 * q + 2], oacc[db][4 * q + 3]} * inv;
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * q) = to_bf16x4(x);
      }
    if (hh == 0) p.lse[(long)(seq0 + row) * p.Hq + h] = (m_run + gq + fast_log2(l_run)) * kLn2;
  }
}

template <int DQK, int DV, int HPW>
static hipError_t launch_pipe_hpw(const FwdParams& p, hipStream_t st) {
  constexpr int BM = 32 * (4 / HPW);
  const int tiles = (p.max_seqlen + BM - 1) / BM;
  const dim3 grid(p.Hq / HPW, tiles, p.num_seqs);
  if (p.G2 != nullptr)
    fwd_pipe_kernel<DQK, DV, true, HPW><<<grid, 256, 0, st>>>(p);
  else
    fwd_pipe_kernel<DQK, DV, false, HPW><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

// Heads per workgroup: 4 when the KV group holds a multiple of 4 query
// heads, else 2, else 1 (the heads of a workgroup share one KV head).
template <int DQK, int DV>
static hipError_t launch_pipe(const FwdParams& p, hipStream_t st) {
  const int grp = p.Hq / p.Hkv;
  if (grp % 4 == 0) return launch_pipe_hpw<DQK, DV, 4>(p, st);
  if (grp % 2 == 0) return launch_pipe_hpw<DQK, DV, 2>(p, st);
  return launch_pipe_hpw<DQK, DV, 1>(p, st);
}

}  // namespace attn
