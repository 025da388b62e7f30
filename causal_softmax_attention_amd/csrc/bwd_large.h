// Two-pass backward, dK/dV pass, for large heads on gfx950: query/key head
// dim 256 with value head dims 256 or 512.
//
// Method (fla issue #1322, Description and the comment of Oct 5): per key
// block, over every query row of the group's heads that sees it,
//   S = Q K^T, P = exp2(S c + G_i - lse_i - G_j) (masked),
//   dP = dO V^T, dS = P (dP - delta_i),
//   dV += P^T dO, dK += dS^T Q (times the softmax scale at the end),
//   dGcol_j = sum_i dS_ij (the key side of the gate gradient).
//
// gfx950 mapping.  With d_v = 512 one wavefront cannot hold the K and V rows
// of its keys and their dK, dV accumulators (288 registers for 16 keys), so
// a workgroup of 8 wavefronts owns 64 keys and splits the work two ways:
//  * phase 1, per 32-row query tile: waves 0-3 hold K of 16 keys each in
//    registers and compute S for them (v_mfma_f32_16x16x32_bf16, Q rows
//    from LDS); waves 4-7 hold V of the same 16-key groups and compute dP
//    (dO rows from LDS), which they hand to their S-wave partner through
//    LDS in fp32.  The S-wave forms P and dS, writes them (bf16, key-major)
//    to LDS and keeps the dS column sums.  The two roles of one key group
//    sit on one SIMD, so the SIMD's MFMA work per tile is the same for all.
//  * phase 2: every wave accumulates dV^T and dK^T for all 64 keys over its
//    eighth of d_v and d_qk (v_mfma_f32_32x32x16_bf16; dO^T and Q^T by
//    ds_read_b64_tr_b16, P and dS from the key-major tiles).
// Q and dO tiles (with the per-row terms and the keys' gate terms) arrive by
// direct global->LDS copies into a two-stage ring, one tile ahead.
// With a dS store (STORE; layout in bwd_ds.h) the S-waves also write dS of
// the band's tiles, the gate's fp32 row sums per 16-key block and the sink
// gradient's per-key sums (sum_i psink_i P_ij dP_ij); the dQ pass is then
// bwd_dq_ds instead of the recomputing kernel below.
#pragma once
#include "bwd_ds.h"
#include "common.h"
#include "kernels.h"

namespace attn {

// Chunk swizzle of the Q and dO tiles (rows of 512 or 1024 bytes; 16-byte
// chunk c of row r is stored at c ^ big_swz(r)).  Row reads (ds_read_b128,
// 32 lanes over 512 bytes: 16 consecutive rows x 2 adjacent chunks) need
// bits 1-4 to differ over 16 consecutive rows; transposed reads
// (ds_read_b64_tr_b16 for 32x32 operands, 32 lanes over 256 bytes: 64 bytes
// of 4 consecutive rows) need bits 2-3 to differ over 4 aligned rows.
// Bits 2-3 = r % 4, bit 1 = (r / 4) % 2, bit 4 = (r / 8) % 2 give both.
__device__ __forceinline__ int big_swz(int r) {
  return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | (((r >> 3) & 1) << 4);
}

// Phase-1 product of one wave: acc[rb] += A(rows rb*16 .. +15) B over NS
// k-steps of 32, A read from a swizzled tile (byte address `base` = tile +
// the lane's row / chunk offset; k-step ks sits at base ^ (ks << 6), which
// leaves the tile base alone because tiles are 1 KB aligned), B = op[ks] in
// registers.  The reads run one chunk of two k-steps ahead of the MFMAs.
template <int NS, int RB>
__device__ __forceinline__ void phase1(uint32_t base, const bf16x8* op, f32x4 (&acc)[2]) {
  constexpr int C = 2, NC = NS / C;
  static_assert(NS % C == 0, "chunks");
  bf16x8 a[2][C][2];
  auto load = [&](int c, int buf) {
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[buf][j][rb] = *reinterpret_cast<const LDS_AS bf16x8*>(
            (uintptr_t)((base + rb * 16 * RB) ^ ((uint32_t)(c * C + j) << 6)));
  };
  load(0, 0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + 1 < NC) load(c + 1, (c + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[rb] = mfma16x16x32(a[c & 1][j][rb], op[c * C + j], acc[rb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int DQK, int DV, bool GATED, bool STORE>
__global__ __launch_bounds__(512) void bwd_dkdv_large_kernel(BwdParams p) {
  constexpr int NW = 8;
  constexpr int BN = 64;              // keys per workgroup
  constexpr int RQ = 32;              // query rows per tile
  constexpr int KSQ = DQK / 32, KSV = DV / 32;   // 16x16x32 k-steps of S, dP
  constexpr int QRB = DQK * 2, ORB = DV * 2;     // bytes per Q / dO row
  constexpr int QBLK = RQ * QRB / 1024, OBLK = RQ * ORB / 1024;   // 1 KB copy blocks
  constexpr int NCV = DV / NW / 32;   // 32-column dV blocks per wave
  constexpr int CK = DQK / NW;        // dK columns per wave
  constexpr int PRB = RQ * 2 + 16;    // key-major P / dS rows, padded (80 bytes)
  static_assert(DQK == 256 && (DV == 256 || DV == 512), "large-head shapes");
  static_assert(QBLK % NW == 0 && OBLK % NW == 0 && CK == 32 && NCV >= 1, "tile split");
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds[2][RQ * QRB];
  __shared__ __attribute__((aligned(1024))) uint8_t o_lds[2][RQ * ORB];
  __shared__ __attribute__((aligned(16))) uint8_t pt_lds[BN * PRB];
  __shared__ __attribute__((aligned(16))) uint8_t dst_lds[BN * PRB];
  __shared__ __attribute__((aligned(16))) f32x4 x_lds[4][2][64];        // dP, S-wave partner's
  __shared__ __attribute__((aligned(16))) float row_lds[2][STORE ? 3 : 2][64];   // row term, delta (, psink)
  __shared__ __attribute__((aligned(16))) float gk_lds[2][64];           // keys' gate terms

  const int kvh = blockIdx.x, n = blockIdx.z, ktile = blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int j0 = ktile * BN;
  if (j0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4, h32 = lane >> 5;
  const int W = p.window;
  const bool is_s = wave < 4;          // S-wave (K) or dP-wave (V) in phase 1
  const int kg = wave & 3;             // 16-key group of phase 1
  const int key = j0 + 16 * kg + li;   // this lane's key in phase 1

  // ---- phase-1 operand: K (S-waves) or V (dP-waves) of the lane's key ----
  bf16x8 op[KSV];
  {
    const bool ok = key < L;
    const long kr = (long)(seq0 + min(key, L - 1)) * p.Hkv + kvh;
    const bf16* src = is_s ? reinterpret_cast<const bf16*>(p.k) + kr * DQK + 8 * g
                           : reinterpret_cast<const bf16*>(p.v) + kr * DV + 8 * g;
    const int ns = is_s ? KSQ : KSV;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks)
      op[ks] = (ok && ks < ns) ? *reinterpret_cast<const bf16x8*>(src + 32 * ks) : bf16x8{};
  }
  f32x16 dv_acc[NCV][2], dk_acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int cb = 0; cb < NCV; ++cb) dv_acc[cb][kb] = f32x16{};
    dk_acc[kb] = f32x16{};
  }

  // ---- iteration space: (head of the group, 32-row query tile) ----
  const int i_end = W > 0 ? min(L, j0 + BN - 1 + W) : L;
  const int nqt = (i_end - j0 + RQ - 1) / RQ;
  const int n_it = grp * nqt;

  // fixed per-lane source offsets of the tile copies (wave w: blocks w, w+8, ...)
  const int qstride = p.Hq * QRB, ostride = p.Hq * ORB;
  int qrow[QBLK / NW], qoff[QBLK / NW], orow[OBLK / NW], ooff[OBLK / NW];
#pragma unroll
  for (int j = 0; j < QBLK / NW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    qrow[j] = o / QRB;
    qoff[j] = qrow[j] * qstride + ((((o % QRB) >> 4) ^ big_swz(qrow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < OBLK / NW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    orow[j] = o / ORB;
    ooff[j] = orow[j] * ostride + ((((o % ORB) >> 4) ^ big_swz(orow[j])) << 4);
  }
  auto fetch = [&](int hg, int qt, int st) {
    const int hh = kvh * grp + hg;
    const int i0 = j0 + qt * RQ;
    const bool tail = i0 + RQ > L;               // uniform: only the last tile clamps
    const long r0 = (long)(seq0 + i0) * p.Hq + hh;
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) + r0 * QRB;
    const uint8_t* ob = reinterpret_cast<const uint8_t*>(p.dO) + r0 * ORB;
    const uint32_t ql = lds_addr(q_lds[st]), ol = lds_addr(o_lds[st]);
#pragma unroll
    for (int j = 0; j < QBLK / NW; ++j) {
      const int over = tail ? max(0, i0 + qrow[j] - (L - 1)) : 0;   // rows past the end re-read the last
      dma16(qb, (uint32_t)(qoff[j] - over * qstride), ql + (wave + NW * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < OBLK / NW; ++j) {
      const int over = tail ? max(0, i0 + orow[j] - (L - 1)) : 0;
      dma16(ob, (uint32_t)(ooff[j] - over * ostride), ol + (wave + NW * j) * 1024);
    }
    if (wave == 0) {
      // per-row terms (head-major), lane l -> row min(i0 + l % RQ, L - 1)
      const uint32_t ro = (uint32_t)((min(i0 + (lane % RQ), L - 1) - i0) * 4);
      const long hr = (long)hh * p.T + seq0 + i0;
      dma4(p.rowt + hr, ro, lds_addr(&row_lds[st][0][0]));
      dma4(p.delta + hr, ro, lds_addr(&row_lds[st][1][0]));
      if constexpr (STORE) {
        if (p.psink != nullptr) dma4(p.psink + hr, ro, lds_addr(&row_lds[st][STORE ? 2 : 0][0]));
      }
    }
    if constexpr (GATED) {
      if (wave == 1) {
        // the block's keys for the tile's head, lane l -> key j0 + l
        const uint32_t ko = (uint32_t)(min(j0 + lane, L - 1) * 4);
        dma4(p.G2 + (long)hh * p.T + seq0, ko, lds_addr(&gk_lds[st][0]));
      }
    }
  };

  // wait for the register loads above before the copies start
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) asm volatile("" :: "v"(op[ks]));

  // ---- per-lane LDS offsets ----
  // phase-1 row reads: row li of a 16-row block, chunk 4 ks + g (XOR of ks << 6)
  const uint32_t q_rd = (uint32_t)(li * QRB + ((g ^ big_swz(li)) << 4));
  const uint32_t o_rd = (uint32_t)(li * ORB + ((g ^ big_swz(li)) << 4));
  // P / dS writes: key 16 kg + li, rows rb * 16 + 4 g .. + 3
  const uint32_t pw = (uint32_t)((16 * kg + li) * PRB + 8 * g);
  // phase-2 B operand: key kb * 32 + l % 32, rows 16 ps + 8 h .. + 7
  const uint32_t pr = (uint32_t)((lane & 31) * PRB + 16 * h32);
  // phase-2 transposed reads: row 16 ps + 8 h + 4 jr + vj, columns cbase + 16 vh + 4 vc
  const int vj = (lane & 15) >> 2, vc = lane & 3, vh = (lane >> 4) & 1;
  uint32_t ot_rd[NCV][2], qt_rd[2];
#pragma unroll
  for (int jr = 0; jr < 2; ++jr) {
    const int r = 8 * h32 + 4 * jr + vj;
#pragma unroll
    for (int cb = 0; cb < NCV; ++cb) {
      const int col = wave * (DV / NW) + 32 * cb + 16 * vh + 4 * vc;
      ot_rd[cb][jr] = (uint32_t)(r * ORB + ((((col * 2) >> 4) ^ big_swz(r)) << 4) + ((col * 2) & 15));
    }
    const int col = wave * CK + 16 * vh + 4 * vc;
    qt_rd[jr] = (uint32_t)(r * QRB + ((((col * 2) >> 4) ^ big_swz(r)) << 4) + ((col * 2) & 15));
  }

  float colsum = 0.f;                  // S-waves: dS column sum of the lane's key (its 4 rows)
  float sinkcol = 0.f;                 // S-waves, dS store: sum of psink_i P_ij dP_ij over the lane's rows
  const bool has_psink = STORE && p.psink != nullptr;
  const bool b3 = (li >> 3) & 1, b2 = (li >> 2) & 1, b1 = (li >> 1) & 1;
  int f_hg = 0, f_qt = 0;
  fetch(0, 0, 0);
  if (++f_qt == nqt) { f_qt = 0; ++f_hg; }
  int it = 0;
  for (int hg = 0; hg < grp; ++hg) {
    for (int qt = 0; qt < nqt; ++qt, ++it) {
      const int st = it & 1;
      wait_vm<0>();
      lds_barrier();   // tile it landed everywhere; tile it-1's LDS is free
      if (it + 1 < n_it) {
        fetch(f_hg, f_qt, st ^ 1);
        if (++f_qt == nqt) { f_qt = 0; ++f_hg; }
      }
      const int i0 = j0 + qt * RQ;
      const uint8_t* ql = q_lds[st];
      const uint8_t* ol = o_lds[st];

      // ---- phase 1: S (S-waves) or dP (dP-waves): C lane = key li, rows rb*16 + 4g + i ----
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 pv[2];
      if (is_s) {
        phase1<KSQ, QRB>(lds_addr(ql) + q_rd, op, acc);
        // P (masked only on tiles that need it) needs only S: formed and
        // stored key-major while the dP-waves finish their longer product
        const bool need_mask = (i0 < j0 + BN - 1) || (W > 0 && i0 + RQ - 1 - j0 >= W) || (i0 + RQ > L) ||
                               (j0 + BN > L);
        const float gk = GATED ? gk_lds[st][16 * kg + li] : 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 rowt = *reinterpret_cast<const f32x4*>(&row_lds[st][0][rb * 16 + 4 * g]);
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[rb][i] = fast_exp2(__builtin_fmaf(acc[rb][i], p.scale_log2, rowt[i] - gk));
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = i0 + rb * 16 + 4 * g + i;
              const bool vis = key < L && row < L && key <= row && (W <= 0 || row - key < W);
              pv[rb][i] = vis ? pv[rb][i] : 0.f;
            }
          }
          *reinterpret_cast<bf16x4*>(pt_lds + pw + rb * 32) = to_bf16x4(pv[rb]);
        }
      } else {
        phase1<KSV, ORB>(lds_addr(ol) + o_rd, op, acc);
        x_lds[kg][0][lane] = acc[0];
        x_lds[kg][1][lane] = acc[1];
      }
      lds_barrier();   // dP of every key group visible

      // ---- S-waves: dS = P (dP - delta), key-major bf16 ----
      if (is_s) {
        f32x4 dsv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 dp = x_lds[kg][rb][lane];
          const f32x4 del = *reinterpret_cast<const f32x4*>(&row_lds[st][1][rb * 16 + 4 * g]);
          f32x4 ds;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ds[i] = pv[rb][i] * (dp[i] - del[i]);
            colsum += ds[i];
          }
          *reinterpret_cast<bf16x4*>(dst_lds + pw + rb * 32) = to_bf16x4(ds);
          dsv[rb] = ds;
          if constexpr (STORE) {
            if (has_psink) {
              const f32x4 ps4 = *reinterpret_cast<const f32x4*>(&row_lds[st][STORE ? 2 : 0][rb * 16 + 4 * g]);
#pragma unroll
              for (int i = 0; i < 4; ++i) sinkcol = __builtin_fmaf(pv[rb][i] * ps4[i], dp[i], sinkcol);
            }
          }
        }
        if constexpr (STORE) {
          // dS tile of (head, row tile i0 / 32, this group's key block), for
          // the band's tiles only (the others hold no visible pair)
          const int rt = i0 / kDsRows, kb = (j0 + 16 * kg) / kDsKeys;
          const int slot = kb - ds_kb_lo(rt, W);
          if (slot >= 0 && slot < p.ds_nslot && kb <= ds_kb_hi(rt, L)) {
            const long t = ds_tile(kvh * grp + hg, ds_grt(seq0, n, rt), slot, p.ds_nrt, p.ds_nslot);
            uint8_t* tb = reinterpret_cast<uint8_t*>(p.ds) + t * kDsTileBytes;
            *reinterpret_cast<bf16x4*>(tb + ds_off(li, 4 * g)) = to_bf16x4(dsv[0]);
            *reinterpret_cast<bf16x4*>(tb + ds_off(li, 16 + 4 * g)) = to_bf16x4(dsv[1]);
            if constexpr (GATED) {
              // fp32 row sums over the block's 16 keys (lanes li): reduce-scatter
              // over lane bits 3, 2, 1, then a pair sum; lane li ends with row
              // 16 b3 + 4 g + 2 b2 + b1
              float a[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float keep = b3 ? dsv[1][j] : dsv[0][j], send = b3 ? dsv[0][j] : dsv[1][j];
                a[j] = keep + dpp_f32<0x140>(send);
              }
              float c[2];
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const float keep = b2 ? a[2 + j] : a[j], send = b2 ? a[j] : a[2 + j];
                c[j] = keep + dpp_f32<0x141>(send);
              }
              const float keep = b1 ? c[1] : c[0], send = b1 ? c[0] : c[1];
              float r = keep + dpp_f32<0x4e>(send);
              r += dpp_f32<0xb1>(r);
              if ((li & 1) == 0) p.ds_rows[t * kDsRows + 16 * b3 + 4 * g + 2 * b2 + b1] = r;
            }
          }
        }
      }
      lds_barrier();   // P and dS of the tile visible

      // ---- phase 2: dV^T += dO^T P, dK^T += Q^T dS over this wave's columns ----
#pragma unroll
      for (int ps = 0; ps < RQ / 16; ++ps) {
        bf16x8 pf[2], df[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pf[kb] = *reinterpret_cast<const bf16x8*>(pt_lds + pr + kb * 32 * PRB + ps * 32);
          df[kb] = *reinterpret_cast<const bf16x8*>(dst_lds + pr + kb * 32 * PRB + ps * 32);
        }
#pragma unroll
        for (int cb = 0; cb < NCV; ++cb) {
          const uint8_t* b = ol + ps * 16 * ORB;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(b + ot_rd[cb][0])),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(b + ot_rd[cb][1])));
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            dv_acc[cb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb], dv_acc[cb][kb], 0, 0, 0);
        }
        {
          const uint8_t* b = ql + ps * 16 * QRB;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(b + qt_rd[0])),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(b + qt_rd[1])));
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            dk_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[kb], dk_acc[kb], 0, 0, 0);
        }
      }
    }
    if (GATED && is_s) {
      // dS column sums of head hg: the 4 lane groups hold 4 rows each of every tile
      const float cs = xgroup_sum(colsum);
      if (g == 0 && key < L) p.dGcol[(long)(kvh * grp + hg) * p.T + seq0 + key] = cs;
      colsum = 0.f;
    }
    if (has_psink && is_s) {
      const float sc = xgroup_sum(sinkcol);
      if (g == 0 && key < L) p.sink_rows[(long)(kvh * grp + hg) * p.T + seq0 + key] = sc;   // per key
      sinkcol = 0.f;
    }
  }

  // ---- store: C lane = key kb*32 + l%32, columns cbase + 8 q + 4 h .. + 3 ----
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int k = j0 + kb * 32 + (lane & 31);
    if (k >= L) continue;
    bf16* dvp = reinterpret_cast<bf16*>(p.dv) + ((long)(seq0 + k) * p.Hkv + kvh) * DV + wave * (DV / NW) + 4 * h32;
    bf16* dkp = reinterpret_cast<bf16*>(p.dk) + ((long)(seq0 + k) * p.Hkv + kvh) * DQK + wave * CK + 4 * h32;
#pragma unroll
    for (int cb = 0; cb < NCV; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = f32x4{dv_acc[cb][kb][4 * q], dv_acc[cb][kb][4 * q + 1], dv_acc[cb][kb][4 * q + 2],
                              dv_acc[cb][kb][4 * q + 3]};
        *reinterpret_cast<bf16x4*>(dvp + 32 * cb + 8 * q) = to_bf16x4(x);
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = f32x4{dk_acc[kb][4 * q], dk_acc[kb][4 * q + 1], dk_acc[kb][4 * q + 2], dk_acc[kb][4 * q + 3]} *
                      p.scale;
      *reinterpret_cast<bf16x4*>(dkp + 8 * q) = to_bf16x4(x);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ pass for the same shapes.  One workgroup of 8 wavefronts per (HPW query
// heads of one KV head, 64 / HPW rows, sequence): 64 (head, row) slots, 16
// per key group of waves.  Per 32-key tile (K and V through a two-stage LDS
// ring):
//  * waves 0-3 hold Q of their 16 slots and compute S^T = K Q^T; waves 4-7
//    hold dO and compute dP^T = V dO^T and hand it over through LDS; the
//    S-wave forms P and dS, keeps the row sums of dS (gate gradient) and of
//    P dP (sink gradient) and writes dS (bf16, slot-major) to LDS;
//  * every wave accumulates dQ^T = K^T dS^T for all 64 slots over its 32
//    columns of d_qk (K^T by ds_read_b64_tr_b16).
template <int DQK, int DV, bool GATED, int HPW>
__global__ __launch_bounds__(512) void bwd_dq_large_kernel(BwdParams p) {
  constexpr int NW = 8;
  constexpr int SLOTS = 64;
  constexpr int BMH = SLOTS / HPW;    // rows per head
  constexpr int BN = 32;              // keys per tile
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int KRB = DQK * 2, VRB = DV * 2;
  constexpr int KBLK = BN * KRB / 1024, VBLK = BN * VRB / 1024;
  constexpr int PRB = BN * 2 + 16;    // slot-major dS rows, padded (80 bytes)
  constexpr int GH = HPW < 2 ? 2 : HPW;
  static_assert(DQK == 256 && (DV == 256 || DV == 512), "large-head shapes");
  static_assert(KBLK % NW == 0 && VBLK % NW == 0 && DQK / NW == 32, "tile split");
  static_assert(HPW == 1 || HPW == 2 || HPW == 4, "heads per workgroup");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][BN * VRB];
  __shared__ __attribute__((aligned(16))) uint8_t ds_lds[SLOTS * PRB];
  __shared__ __attribute__((aligned(16))) f32x4 x_lds[4][2][64];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][GH][BN];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4, h32 = lane >> 5;
  const int grp = p.Hq / p.Hkv;
  const int nchunk = p.Hq / HPW;
  const int hx = (nchunk % 8 == 0) ? (blockIdx.x % 8) * (nchunk / 8) + blockIdx.x / 8 : blockIdx.x;
  // uniform values computed with vector divides: pinned to scalar registers
  // (the copy bases built from them must be SGPRs)
  const int h0 = __builtin_amdgcn_readfirstlane(hx * HPW);
  const int kvh = __builtin_amdgcn_readfirstlane(h0 / grp);
  const int n = blockIdx.z;
  const int tile = gridDim.y - 1 - blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int i0 = tile * BMH;
  if (i0 >= L) return;
  const int W = p.window;
  const bool is_s = wave < 4;
  const int kg = wave & 3;            // slot group: slots 16 kg .. 16 kg + 15
  const int hw = h0 + kg % HPW;       // its head
  const int r0 = i0 + 16 * (kg / HPW);
  const int r_last = min(r0 + 16, L) - 1;
  const int row = r0 + li;

  // ---- phase-1 operand: Q (S-waves) or dO (dP-waves) of the lane's row ----
  bf16x8 op[KSV];
  float lse2 = 0.f, dlt = 0.f, gq = 0.f;
  {
    const bool ok = row < L;
    const long ri = (long)(seq0 + min(row, L - 1)) * p.Hq + hw;
    const bf16* src = is_s ? reinterpret_cast<const bf16*>(p.q) + ri * DQK + 8 * g
                           : reinterpret_cast<const bf16*>(p.dO) + ri * DV + 8 * g;
    const int ns = is_s ? KSQ : KSV;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks)
      op[ks] = (ok && ks < ns) ? *reinterpret_cast<const bf16x8*>(src + 32 * ks) : bf16x8{};
    if (is_s && ok) {
      lse2 = p.lse[ri] * kLog2e;
      dlt = p.delta[(long)hw * p.T + seq0 + row];
      if constexpr (GATED) gq = p.G2[(long)hw * p.T + seq0 + row];
    }
  }
  f32x16 dq_acc[2] = {f32x16{}, f32x16{}};
  float rowsum = 0.f, pdp = 0.f;

  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BMH);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + ((long)seq0 * p.Hkv + kvh) * VRB;
  const int kstride = p.Hkv * KRB, vstride = p.Hkv * VRB;
  int krow[KBLK / NW], koff[KBLK / NW], vrow[VBLK / NW], voff[VBLK / NW];
#pragma unroll
  for (int j = 0; j < KBLK / NW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    krow[j] = o / KRB;
    koff[j] = krow[j] * kstride + ((((o % KRB) >> 4) ^ big_swz(krow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < VBLK / NW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    vrow[j] = o / VRB;
    voff[j] = vrow[j] * vstride + ((((o % VRB) >> 4) ^ big_swz(vrow[j])) << 4);
  }
  auto fetch = [&](int t, int st) {
    const int j0 = t * BN;
    const bool tail = j0 + BN > L;
    const uint8_t* kb = sgpr_ptr(kbase + (long)j0 * kstride);
    const uint8_t* vb = sgpr_ptr(vbase + (long)j0 * vstride);
    const uint32_t kl = lds_addr(k_lds[st]), vl = lds_addr(v_lds[st]);
#pragma unroll
    for (int j = 0; j < KBLK / NW; ++j) {
      const int over = tail ? max(0, j0 + krow[j] - (L - 1)) : 0;   // rows past the end re-read the last
      dma16(kb, (uint32_t)(koff[j] - over * kstride), kl + (wave + NW * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < VBLK / NW; ++j) {
      const int over = tail ? max(0, j0 + vrow[j] - (L - 1)) : 0;
      dma16(vb, (uint32_t)(voff[j] - over * vstride), vl + (wave + NW * j) * 1024);
    }
    if constexpr (GATED) {
      // keys' gate terms of two heads per copy: lane l -> head 2 w + l / 32, key l % 32
      if (2 * wave < HPW) {
        const float* gb = sgpr_ptr(p.G2 + (long)(h0 + 2 * wave) * p.T + seq0);
        const int hsel = min(2 * wave + h32, HPW - 1) - 2 * wave;
        const uint32_t go = (uint32_t)((hsel * p.T + min(j0 + (lane & 31), L - 1)) * 4);
        dma4(gb, go, __builtin_amdgcn_readfirstlane(lds_addr(&gk_lds[st][2 * wave][0])));
      }
    }
  };

#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) asm volatile("" :: "v"(op[ks]));
  asm volatile("" :: "v"(lse2), "v"(dlt), "v"(gq));

  // ---- per-lane LDS offsets ----
  const uint32_t k_rd = (uint32_t)(li * KRB + ((g ^ big_swz(li)) << 4));
  const uint32_t v_rd = (uint32_t)(li * VRB + ((g ^ big_swz(li)) << 4));
  const uint32_t dsw = (uint32_t)((16 * kg + li) * PRB + 8 * g);        // slot, keys kb*16 + 4g
  const uint32_t dsr = (uint32_t)((lane & 31) * PRB + 16 * h32);        // slot sb*32 + l%32, keys 16ps + 8h
  const int vj = (lane & 15) >> 2, vc = lane & 3, vh = (lane >> 4) & 1;
  uint32_t kt_rd[2];
#pragma unroll
  for (int jr = 0; jr < 2; ++jr) {
    const int r = 8 * h32 + 4 * jr + vj;
    const int col = wave * 32 + 16 * vh + 4 * vc;
    kt_rd[jr] = (uint32_t)(r * KRB + ((((col * 2) >> 4) ^ big_swz(r)) << 4) + ((col * 2) & 15));
  }

  const float c = p.scale_log2;
  const float rowt = gq - lse2;
  if (t_begin < t_end) fetch(t_begin, 0);
  for (int t = t_begin; t < t_end; ++t) {
    const int st = (t - t_begin) & 1;
    const int j0 = t * BN;
    wait_vm<0>();
    lds_barrier();   // tile t landed everywhere; tile t-1's LDS is free
    if (t + 1 < t_end) fetch(t + 1, st ^ 1);

    // ---- phase 1: C lane = slot li, keys kb*16 + 4g + i ----
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 pv[2];
    if (is_s) {
      phase1<KSQ, KRB>(lds_addr(k_lds[st]) + k_rd, op, acc);
      // P needs only S: formed while the dP-waves finish their longer product
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + 15);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 gk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(&gk_lds[st][kg % HPW][kb * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[kb][i] = fast_exp2(__builtin_fmaf(acc[kb][i], c, rowt - gk[i]));
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j0 + kb * 16 + 4 * g + i;
            const bool vis = key <= row && key < L && row < L && (W <= 0 || row - key < W);
            pv[kb][i] = vis ? pv[kb][i] : 0.f;
          }
        }
      }
    } else {
      phase1<KSV, VRB>(lds_addr(v_lds[st]) + v_rd, op, acc);
      x_lds[kg][0][lane] = acc[0];
      x_lds[kg][1][lane] = acc[1];
    }
    lds_barrier();

    if (is_s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x4 dp = x_lds[kg][kb][lane];
        f32x4 ds;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ds[i] = pv[kb][i] * (dp[i] - dlt);
          rowsum += ds[i];
          pdp += pv[kb][i] * dp[i];
        }
        *reinterpret_cast<bf16x4*>(ds_lds + dsw + kb * 32) = to_bf16x4(ds);
      }
    }
    lds_barrier();

    // ---- phase 2: dQ^T += K^T dS^T over this wave's 32 columns ----
#pragma unroll
    for (int ps = 0; ps < BN / 16; ++ps) {
      const uint8_t* b = k_lds[st] + ps * 16 * KRB;
      const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(b + kt_rd[0])),
                              lds_read_tr16(reinterpret_cast<const bf16*>(b + kt_rd[1])));
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 df = *reinterpret_cast<const bf16x8*>(ds_lds + dsr + sb * 32 * PRB + ps * 32);
        dq_acc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df, dq_acc[sb], 0, 0, 0);
      }
    }
  }

  if (is_s) {
    const float rs = xgroup_sum(rowsum);
    const float sp = xgroup_sum(pdp);
    if (g == 0 && row < L) {
      const long hm = (long)hw * p.T + seq0 + row;   // head-major
      if (GATED) p.dGrow[hm] = rs;
      if (p.sink) p.sink_rows[hm] = fast_exp2(p.sink[hw] * kLog2e - lse2) * sp;
    }
  }
  // ---- store: C lane = slot sb*32 + l%32, columns 32 w + 8 q + 4 h .. + 3 ----
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int slot = sb * 32 + (lane & 31);
    const int ws = slot >> 4;
    const int sh = h0 + ws % HPW;
    const int srow = i0 + 16 * (ws / HPW) + (slot & 15);
    if (srow >= L) continue;
    bf16* dqp = reinterpret_cast<bf16*>(p.dq) + ((long)(seq0 + srow) * p.Hq + sh) * DQK + wave * 32 + 4 * h32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = f32x4{dq_acc[sb][4 * q], dq_acc[sb][4 * q + 1], dq_acc[sb][4 * q + 2], dq_acc[sb][4 * q + 3]} *
                      p.scale;
      *reinterpret_cast<bf16x4*>(dqp + 8 * q) = to_bf16x4(x);
    }
  }
}

template <int DQK, int DV, int HPW>
hipError_t launch_dq_large_hpw(const BwdParams& p, hipStream_t st) {
  constexpr int BMH = 64 / HPW;
  const dim3 grid(p.Hq / HPW, (p.max_seqlen + BMH - 1) / BMH, p.num_seqs);
  if (p.G2) bwd_dq_large_kernel<DQK, DV, true, HPW><<<grid, 512, 0, st>>>(p);
  else bwd_dq_large_kernel<DQK, DV, false, HPW><<<grid, 512, 0, st>>>(p);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_dq_large_t(const BwdParams& p, hipStream_t st) {
  const int grp = p.Hq / p.Hkv;
  if (grp % 4 == 0) return launch_dq_large_hpw<DQK, DV, 4>(p, st);
  if (grp % 2 == 0) return launch_dq_large_hpw<DQK, DV, 2>(p, st);
  return launch_dq_large_hpw<DQK, DV, 1>(p, st);
}

template <int DQK, int DV>
hipError_t launch_dkdv_large_t(const BwdParams& p, hipStream_t st) {
  const dim3 grid(p.Hkv, (p.max_seqlen + 63) / 64, p.num_seqs);
  if (p.ds != nullptr) {
    if (p.G2) bwd_dkdv_large_kernel<DQK, DV, true, true><<<grid, 512, 0, st>>>(p);
    else bwd_dkdv_large_kernel<DQK, DV, false, true><<<grid, 512, 0, st>>>(p);
  } else {
    if (p.G2) bwd_dkdv_large_kernel<DQK, DV, true, false><<<grid, 512, 0, st>>>(p);
    else bwd_dkdv_large_kernel<DQK, DV, false, false><<<grid, 512, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace attn
