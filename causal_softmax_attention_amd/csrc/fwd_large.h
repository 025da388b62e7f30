// Packed variable-length causal attention forward for large heads on
// gfx950: value heads of 256 or 512 (any query/key head dim), and query/key
// heads of 256 with value heads of 64 or 128.
//
// Method (fla issue #1322, Description): the same definition as the other
// forward kernels (GQA, gate bias G_i - G_j, sliding window, sink logit,
// unequal query/key and value head dims up to 512); fp32 scores from bf16
// operands, bf16 P in the PV product, O rounded to bf16, lse in fp32.
//
// gfx950 mapping: the O tile of a 512-wide value head does not fit one
// wave's registers for more than 16 query rows, and with 16 rows per wave
// every K and V operand read from LDS would feed a single MFMA, which makes
// such a layout LDS-bound.  Here the work of a workgroup is split two ways:
//  * NW wavefronts (8 for d_v >= 256, d_v / 32 below), 16 NW (query head,
//    row) slots: HPW heads of one KV head (GQA-packed) x 16 NW / HPW rows.
//    Wave w owns slots 16 w .. 16 w + 15: it computes S = Q K^T for them
//    (v_mfma_f32_16x16x32_bf16, Q in registers), the online softmax (max,
//    lazy rescale, exp, row sum) and writes P (bf16) and its rescale factors
//    to LDS.
//  * then every wave computes O for all slots over its 1 / NW of d_v:
//    O^T += V^T P^T with v_mfma_f32_32x32x16_bf16 (V^T from
//    ds_read_b64_tr_b16, P^T rows from the padded P tile), so each V
//    fragment feeds 16 NW / 32 MFMAs and each P fragment one per 32 columns.
//    Before accumulating it applies the rescale factors the owners wrote.
// The tile loop is software pipelined: iteration u forms S, the softmax and
// P of tile u + 1 (P and its rescale factors into one of two LDS buffers)
// and accumulates the PV of tile u from the other buffer, half of it before
// the softmax and half between its exponentials.  One barrier per 32-key
// tile publishes P(u + 1), the K of tile u + 1 and the V of tile u; K and V
// have rings of their own, so tile u + 2's K and tile u + 1's V can be copied
// as soon as the barrier has retired the reads of K(u) and V(u - 1).
// K and V tiles arrive by direct global->LDS copies into a two-stage ring;
// K uses the row-read swizzle of tile_swz, V a swizzle that keeps the rows
// of a transposed read on different bank segments; P rows are
// padded to 80 bytes, so the 32 rows of a P read fall on different banks.
#pragma once
#include "common.h"
#include "kernels.h"

namespace attn {

// Wavefronts per workgroup: one per 32 value columns, at most 8.
template <int DV>
constexpr int large_waves() { return DV >= 256 ? 8 : DV / 32; }

template <int DQK, int DV, bool GATED, int HPW>
__global__ __launch_bounds__(64 * large_waves<DV>()) void fwd_large_kernel(FwdParams p) {
  constexpr int NW = large_waves<DV>(); // wavefronts
  constexpr int SLOTS = 16 * NW;        // (head, row) slots of the workgroup
  constexpr int BMH = SLOTS / HPW;      // rows per head
  constexpr int BN = 32;                // keys per tile
  constexpr int KB = BN / 16;           // 16-key blocks of S
  constexpr int KS = DQK / 32;          // QK k-steps
  constexpr int DVW = DV / NW;          // value columns per wave in PV
  constexpr int NDB = DVW / 32;         // 32-wide column blocks per wave
  constexpr int NRB = SLOTS / 32;       // 32-slot row blocks
  constexpr int PS = BN / 16;           // PV k-steps
  constexpr int KRB = DQK * 2, VRB = DV * 2;
  constexpr int PRB = BN * 2 + 16;      // P row bytes, padded (80: rows land on distinct banks)
  constexpr int KBLK = BN * KRB / 1024, VBLK = BN * VRB / 1024;   // 1 KB copy blocks per tile
  static_assert(NDB >= 1 && DVW % 32 == 0, "value columns per wave");
  static_assert(KBLK >= 1 && VBLK % NW == 0, "copy blocks");
  static_assert((HPW == 1 || HPW == 2 || HPW == 4) && HPW <= NW, "heads per workgroup");
  static_assert(NW >= 2 && NRB >= 1, "workgroup shape");
  constexpr int GH = HPW < 2 ? 2 : HPW;  // gate rows held (one copy fills two heads)
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][BN * VRB];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2][SLOTS * PRB];
  __shared__ __attribute__((aligned(16))) float alpha_lds[2][SLOTS];
  __shared__ __attribute__((aligned(16))) float l_lds[SLOTS];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][GH][BN];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int grp = p.Hq / p.Hkv;
  const int nchunk = p.Hq / HPW;
  const int hx = (nchunk % 8 == 0) ? (blockIdx.x % 8) * (nchunk / 8) + blockIdx.x / 8 : blockIdx.x;
  const int h0 = hx * HPW;              // first head of the workgroup
  const int kvh = h0 / grp;
  const int n = blockIdx.z;
  const int tile = gridDim.y - 1 - blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int i0 = tile * BMH;
  if (i0 >= L) return;
  const int W = p.window;
  const float c = p.scale_log2;

  // ---- this wave's own slots: head hw, rows r0 .. r0 + 15 ----
  const int hw = h0 + wave % HPW;
  const int r0 = i0 + 16 * (wave / HPW);
  const int r_last = min(r0 + 16, L) - 1;
  const int row = r0 + li;
  bf16x8 qop[KS];
  float gq = 0.f;
  if (row < L) {
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + ((long)(seq0 + row) * p.Hq + hw) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
    if constexpr (GATED) gq = p.G2[(long)hw * p.T + seq0 + row];
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = bf16x8{};
  }
  const float sink2 = p.sink ? p.sink[hw] * kLog2e : kNegBig;
  float m_run = p.sink ? sink2 - gq : kNegBig;   // kept without the row's gate term gq
  float l_run = p.sink && g == 0 ? 1.f : 0.f;   // per-lane parts of the row sum

  // ---- O of all slots over this wave's value columns ----
  f32x16 oacc[NDB][NRB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) oacc[db][rb] = f32x16{};

  // ---- key range of the workgroup ----
  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BMH);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;

  // ---- tile copies: wave w copies the 1 KB blocks w, w + 8, ... ----
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + ((long)seq0 * p.Hkv + kvh) * VRB;
  const int kstride = p.Hkv * KRB, vstride = p.Hkv * VRB;
  // V chunk swizzle: a transposed read covers 64 bytes of 4 consecutive
  // rows, served over 256 bytes of banks.  Rows of 256 bytes or more: chunk
  // bits 2-3 from r % 4 put the 4 rows on 4 different 64-byte segments.
  // 128-byte rows (8 chunks): only rows 2 apart share banks, so bit 2 from
  // (r / 2) % 2 separates them.  Both depend only on r % 4, which the
  // per-lane offsets below rely on.
  auto v_swz = [](int r) { return VRB >= 256 ? (r & 3) << 2 : ((r >> 1) & 1) << 2; };
  // copies of tile t_begin + u: K (and the keys' gate terms) into K stage
  // u & 1, V into V stage u & 1
  auto fetch_k = [&](int u) {
    const int j0 = (t_begin + u) * BN, st = u & 1;
    const bool tail = j0 + BN > L;
    const uint8_t* kb = kbase + (long)j0 * kstride;
#pragma unroll
    for (int jj = 0; jj < (KBLK + NW - 1) / NW; ++jj) {
      const int j = wave + NW * jj;
      if (KBLK % NW != 0 && j >= KBLK) break;         // uniform
      const int o = j * 1024 + lane * 16;
      const int r = o / KRB;
      const int rr = tail ? min(r, L - 1 - j0) : r;   // rows past the end re-read the last row
      const uint32_t off = (uint32_t)(rr * kstride + ((((o % KRB) >> 4) ^ tile_swz<KRB>(r)) << 4));
      dma16(kb, off, __builtin_amdgcn_readfirstlane(lds_addr(k_lds[st]) + j * 1024));
    }
    if constexpr (GATED) {
      // gate terms of two heads per copy: lane l -> head 2 w + l / 32, key l % 32
      if (2 * wave < HPW) {
        const float* gb = p.G2 + (long)(h0 + 2 * wave) * p.T + seq0;   // wave-uniform base
        const int hsel = min(2 * wave + (lane >> 5), HPW - 1) - 2 * wave;
        const uint32_t go = (uint32_t)((hsel * p.T + min(j0 + (lane & 31), L - 1)) * 4);
        dma4(gb, go, __builtin_amdgcn_readfirstlane(lds_addr(&gk_lds[st][2 * wave][0])));
      }
    }
  };
  auto fetch_v = [&](int u) {
    const int j0 = (t_begin + u) * BN, st = u & 1;
    const bool tail = j0 + BN > L;
    const uint8_t* vb = vbase + (long)j0 * vstride;
#pragma unroll
    for (int jj = 0; jj < VBLK / NW; ++jj) {
      const int j = wave + NW * jj;
      const int o = j * 1024 + lane * 16;
      const int r = o / VRB;
      const int rr = tail ? min(r, L - 1 - j0) : r;
      const uint32_t off = (uint32_t)(rr * vstride + ((((o % VRB) >> 4) ^ v_swz(r)) << 4));
      dma16(vb, off, __builtin_amdgcn_readfirstlane(lds_addr(v_lds[st]) + j * 1024));
    }
  };

  // ---- per-lane LDS offsets ----
  // K fragment (16-key block kb, k-step ks): row kb*16 + li, chunk 4 ks + g
  uint32_t k_lane[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_lane[ks] = (uint32_t)tile_off<KRB>(li, 64 * ks + 16 * g);
  // P write: slot 16 w + li, keys kb*16 + 4g .. + 3 (8 bytes)
  const uint32_t p_wr = (uint32_t)((16 * wave + li) * PRB + 8 * g);
  // P^T fragment (row block rb, k-step s): slot rb*32 + l%32, keys 16 s + 8 h .. + 7
  const int hh2 = lane >> 5;
  const uint32_t p_rd = (uint32_t)((lane & 31) * PRB + 16 * hh2);
  // V^T fragment (k-step s, column block db, read jr): row 16 s + 8 h + 4 jr + j,
  // column wave*DVW + db*32 + 16 half + 4 cc (j = (l%16)/4, cc = l%4, half = (l/16)%2)
  const int vj = (lane & 15) >> 2, vcc = lane & 3, vhalf = (lane >> 4) & 1;
  uint32_t v_lane[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int r = 8 * hh2 + vj;   // row within the 16-key step (r % 4 = vj)
    const int col = wave * DVW + db * 32 + 16 * vhalf + 4 * vcc;
    const int ch = (col * 2) >> 4;
    v_lane[db] = (uint32_t)(r * VRB + ((ch ^ v_swz(r)) << 4) + ((col * 2) & 15));
  }

  // ---- S of tile t_begin + u for this wave's 16 slots (C lane: row li, keys 4g + i) ----
  auto s_tile = [&](int u, f32x4 (&s)[KB]) {
    const uint8_t* kt = k_lds[u & 1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)   // the key blocks' chains alternate
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + k_lane[ks] + kb * 16 * KRB);
        s[kb] = mfma16x16x32(a, qop[ks], s[kb]);
      }
  };
  // ---- bias, mask, online softmax; P and the rescale factor into buffer u & 1 ----
  auto softmax_tile = [&](int u, f32x4 (&s)[KB], auto&& between) {
    const int j0 = (t_begin + u) * BN, st = u & 1;
    const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) || (r_last < r0 + 15);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x4 gk = {0.f, 0.f, 0.f, 0.f};
      if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(&gk_lds[st][wave % HPW][kb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kb][i] = GATED ? __builtin_fmaf(s[kb][i], c, -gk[i]) : s[kb][i] * c;
    }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j0 + kb * 16 + 4 * g + i;
          const bool vis = key <= row && key < L && (W <= 0 || row - key < W);
          s[kb][i] = vis ? s[kb][i] : -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
    // lazy rescale, without a branch (so that the exponentials can be
    // scheduled between the MFMAs of the other tile's PV): the running max
    // moves only when some lane's own max passes it by more than the slack,
    // which is when the row max does
    between();   // the other tile's MFMAs that the exponentials can hide behind
    const float mg = xgroup_max(mx);
    const float m_new = __any(mx > m_run + kRescaleSlack) ? fmaxf(m_run, mg) : m_run;
    const float alpha = m_new != m_run ? fast_exp2(m_run - m_new) : 1.f;
    l_run *= alpha;
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = fast_exp2(s[kb][i] - m_run);
      rs += (e[0] + e[1]) + (e[2] + e[3]);
      *reinterpret_cast<bf16x4*>(p_lds[st] + p_wr + kb * 32) = to_bf16x4(e);
    }
    l_run += rs;   // the lane groups' parts are added after the loop
    if (g == 0) alpha_lds[st][16 * wave + li] = alpha;
  };
  // ---- O^T += V^T P^T of tile t_begin + u over this wave's columns, for all slots ----
  auto o_rescale = [&](int u) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float a = alpha_lds[u & 1][rb * 32 + (lane & 31)];
      if (__builtin_expect(__any(a != 1.f), 0)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][rb] *= a;
      }
    }
  };
  auto pv_tile = [&](int u, int ps_lo, int ps_hi) {   // k-steps ps_lo .. ps_hi - 1
    const uint8_t* pt = p_lds[u & 1];
    const uint8_t* vt = v_lds[u & 1];
#pragma unroll
    for (int ps = ps_lo; ps < ps_hi; ++ps) {
      bf16x8 pf[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        pf[rb] = *reinterpret_cast<const bf16x8*>(pt + p_rd + rb * 32 * PRB + ps * 32);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint8_t* vb = vt + v_lane[db] + 16 * ps * VRB;
        const bf16x8 vf = concat(lds_read_tr16(reinterpret_cast<const bf16*>(vb)),
                                 lds_read_tr16(reinterpret_cast<const bf16*>(vb + 4 * VRB)));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          oacc[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb], oacc[db][rb], 0, 0, 0);
      }
    }
  };

  // ---- tile loop, software pipelined across waves and tiles: iteration u
  // computes S and P of tile u + 1 and the PV of tile u, so one barrier per
  // tile publishes P(u + 1) and retires the reads of tiles u (K) and u - 1 (V) ----
  const int NT = t_end - t_begin;
  fetch_k(0);
  fetch_v(0);
  if (NT > 1) fetch_k(1);
  wait_vm<0>();
  lds_barrier();
  {
    f32x4 s[KB];
    s_tile(0, s);
    softmax_tile(0, s, [] {});
  }
  for (int u = 0; u + 1 < NT; ++u) {
    wait_vm<0>();
    lds_barrier();   // K(u + 1) and V(u) landed, P(u) visible; tile u - 1 fully read
    if (u + 2 < NT) fetch_k(u + 2);   // into the stage of K(u), read in the last iteration
    fetch_v(u + 1);                   // into the stage of V(u - 1), likewise
    o_rescale(u);
    f32x4 s[KB];
    s_tile(u + 1, s);
    pv_tile(u, 0, PS / 2);
    softmax_tile(u + 1, s, [&] { pv_tile(u, PS / 2, PS); });
  }
  wait_vm<0>();
  lds_barrier();   // P of the last tile visible
  o_rescale(NT - 1);
  pv_tile(NT - 1, 0, PS);

  // ---- finalize: row sums of every slot from their owners; O = acc / l ----
  l_run = xgroup_sum(l_run);
  lds_barrier();
  if (g == 0) l_lds[16 * wave + li] = l_run;
  if (g == 0 && row < L) p.lse[(long)(seq0 + row) * p.Hq + hw] = (m_run + gq + fast_log2(l_run)) * kLn2;
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int slot = rb * 32 + (lane & 31);
    const int ws = slot >> 4;                      // owner wave of the slot
    const int sh = h0 + ws % HPW;
    const int srow = i0 + 16 * (ws / HPW) + (slot & 15);
    if (srow >= L) continue;
    const float inv = 1.0f / l_lds[slot];
    bf16* op = reinterpret_cast<bf16*>(p.o) + ((long)(seq0 + srow) * p.Hq + sh) * DV + wave * DVW + 4 * hh2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = f32x4{oacc[db][rb][4 * q], oacc[db][rb][4 * q + 1], oacc[db][rb][4 * q + 2],
                              oacc[db][rb][4 * q + 3]} * inv;
        *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * q) = to_bf16x4(x);
      }
  }
}

template <int DQK, int DV, int HPW>
static hipError_t launch_large_hpw(const FwdParams& p, hipStream_t st) {
  constexpr int NW = large_waves<DV>();
  constexpr int BMH = 16 * NW / HPW;
  const int tiles = (p.max_seqlen + BMH - 1) / BMH;
  const dim3 grid(p.Hq / HPW, tiles, p.num_seqs);
  if (p.G2 != nullptr)
    fwd_large_kernel<DQK, DV, true, HPW><<<grid, 64 * NW, 0, st>>>(p);
  else
    fwd_large_kernel<DQK, DV, false, HPW><<<grid, 64 * NW, 0, st>>>(p);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_large(const FwdParams& p, hipStream_t st) {
  constexpr int NW = large_waves<DV>();
  const int grp = p.Hq / p.Hkv;
  if constexpr (NW >= 4) {
    if (grp % 4 == 0) return launch_large_hpw<DQK, DV, 4>(p, st);
  }
  if (grp % 2 == 0) return launch_large_hpw<DQK, DV, 2>(p, st);
  return launch_large_hpw<DQK, DV, 1>(p, st);
}

}  // namespace attn
