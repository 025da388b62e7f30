// Deterministic two-pass backward for gfx950 (no atomics anywhere): the
// kernels and their launch sequence, instantiated per query/key head dim in
// bwd2.hip, bwd2_qk128.hip and bwd2_qk256.hip.
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
//
// With a dS store (STORE; layout in bwd_ds.h) the dK/dV pass also writes dS
// and, for the gate, its fp32 row sums per 16-key block, and accumulates the
// sink gradient per key (sum_i psink_i P_ij dP_ij, a column sum like the
// gate's); the dQ pass is then bwd_dq_ds (bwd_dq_ds.h), which reads dS
// instead of forming S and dP again.
#pragma once
#include "bwd_dq_ds.h"
#include "bwd_ds.h"
#include "common.h"
#include "kernels.h"

namespace attn {

// Tile shapes of the head-dim 64 / 128 kernels (measured on config-sized
// workloads: 16 keys per dK/dV wave keep three waves per SIMD; 32 query rows
// per dQ wave; a two-stage Q/dO ring, three stages measured slower).
constexpr int kBwdKwSmall = 16, kBwdRwSmall = 32, kBwdNstDkdv = 2;


// ---------------------------------------------------------------------------
// dK/dV pass.  Each wave keeps KW keys of K and V in registers and walks the
// query tiles (RQ rows) of every query head of its KV group.  The Q and dO
// tiles (and the per-row lse, delta and gate terms) reach LDS by direct
// copies into a two-stage ring of swizzled tiles, one tile ahead of the
// math; rows past the end re-read the last row (finite) and are masked.
// (three waves per SIMD for the head dims that fit them: the dS store's
// extra registers would otherwise tip the 128/128 kernel over 168)
template <int DQK, int DV, int KW, bool GATED, bool STORE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DQK + DV <= 256 ? 3 : 1)))
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int RQ = 32;              // query rows per tile
  constexpr int KBW = KW / 16;        // 16-key blocks per wave
  constexpr int BNW = 4 * KW;         // keys per workgroup
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int DBQ = DQK / 16, DBV = DV / 16;
  constexpr int QRB = DQK * 2, ORB = DV * 2;   // bytes per Q / dO row
  constexpr int QPW = RQ * QRB / 4096, OPW = RQ * ORB / 4096;   // 1 KB blocks per wave
  static_assert(QPW * 4096 == RQ * QRB && OPW * 4096 == RQ * ORB, "tile must split into 4 x k 1 KB blocks");
  constexpr int NSQ = kBwdNstDkdv;    // ring stages (tiles in flight: NSQ - 1)
  static_assert(NSQ >= 2 && NSQ <= 3, "ring depth");
  // copies per tile issued by every wave (wave 0 adds the per-row terms):
  // the exact count of the later tiles' copies a wave waits past
  constexpr int LPT = QPW + OPW + (GATED ? 1 : 0);
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds[NSQ][RQ * QRB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds[NSQ][RQ * ORB];
  static_assert(!STORE || KW == kDsKeys, "a wave's keys are one dS key block");
  // row term, delta (and psink with a dS store); lanes >= RQ repeat
  __shared__ __attribute__((aligned(16))) float row_lds[NSQ][STORE ? 3 : 2][64];
  __shared__ __attribute__((aligned(16))) float gk_lds[NSQ][4][64];    // per wave: its keys' gate terms

  const int kvh = xcd_remap(blockIdx.x, p.Hkv), n = blockIdx.z, ktile = blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int j0 = ktile * BNW;
  if (j0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
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

  // Flattened iteration over (query head of the group, RQ-row query tile).
  const int i_end = W > 0 ? min(L, j0 + BNW - 1 + W) : L;
  const int nqt = (i_end - j0 + RQ - 1) / RQ;
  const int n_it = grp * nqt;

  // fixed per-lane source offsets of the tile copies
  const int qstride = p.Hq * QRB, ostride = p.Hq * ORB;
  int qrow[QPW], qoff[QPW], orow[OPW], ooff[OPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    qrow[j] = o / QRB;
    qoff[j] = qrow[j] * qstride + ((((o % QRB) >> 4) ^ tile_swz<QRB>(qrow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < OPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    orow[j] = o / ORB;
    ooff[j] = orow[j] * ostride + ((((o % ORB) >> 4) ^ tile_swz<ORB>(orow[j])) << 4);
  }
  // iteration (head hg of the group, query tile qt); the counters advance
  // by one per iteration (no division in the loop)
  auto advance = [&](int& hg, int& qt) {
    if (++qt == nqt) { qt = 0; ++hg; }
  };
  auto fetch = [&](int hg, int qt, int st) {
    const int hh = kvh * grp + hg;
    const int i0 = j0 + qt * RQ;
    const bool tail = i0 + RQ > L;               // uniform: only the last tile clamps
    const long r0 = (long)(seq0 + i0) * p.Hq + hh;   // (token, head) row of the tile's first query
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(p.q) + r0 * QRB;
    const uint8_t* ob = reinterpret_cast<const uint8_t*>(p.dO) + r0 * ORB;
    const uint32_t ql = lds_addr(q_lds[st]), ol = lds_addr(do_lds[st]);
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int over = tail ? max(0, i0 + qrow[j] - (L - 1)) : 0;
      dma16(qb, (uint32_t)(qoff[j] - over * qstride), ql + (wave + 4 * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < OPW; ++j) {
      const int over = tail ? max(0, i0 + orow[j] - (L - 1)) : 0;
      dma16(ob, (uint32_t)(ooff[j] - over * ostride), ol + (wave + 4 * j) * 1024);
    }
    if (wave == 0) {
      // per-row terms (head-major: the tile's rows are contiguous),
      // lane l -> row min(i0 + l % RQ, L - 1)
      const uint32_t ro = (uint32_t)((min(i0 + (lane % RQ), L - 1) - i0) * 4);
      const long hr = (long)hh * p.T + seq0 + i0;
      dma4(p.rowt + hr, ro, lds_addr(&row_lds[st][0][0]));
      dma4(p.delta + hr, ro, lds_addr(&row_lds[st][1][0]));
      if constexpr (STORE) {
        if (p.psink != nullptr) dma4(p.psink + hr, ro, lds_addr(&row_lds[st][STORE ? 2 : 0][0]));
      }
    }
    if constexpr (GATED) {
      // this wave's keys for the tile's head, lane l -> key jw + l % KW
      const uint32_t ko = (uint32_t)(min(jw + (lane % KW), L - 1) * 4);
      dma4(p.G2 + (long)hh * p.T + seq0, ko, lds_addr(&gk_lds[st][wave][0]));
    }
  };

  // wait for the register loads above before the copies start, so that the
  // compiler's own wait for them does not land inside the loop
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) asm volatile("" :: "v"(kop[kb][ks]));
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) asm volatile("" :: "v"(vop[kb][ks]));
  }

  int f_hg = 0, f_qt = 0;   // the next tile to fetch
#pragma unroll
  for (int s0 = 0; s0 < NSQ - 1; ++s0)
    if (s0 < n_it) {
      fetch(f_hg, f_qt, s0);
      advance(f_hg, f_qt);
    }
  float colsum[KBW], sinkcol[KBW];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) colsum[kb] = sinkcol[kb] = 0.f;
  // dS store: the lane-dependent selections of the row-sum reduction (lane
  // bits 3, 2, 1 pick the half kept at each step) and the sink switch
  const bool b3 = (li >> 3) & 1, b2 = (li >> 2) & 1, b1 = (li >> 1) & 1;
  const bool has_psink = STORE && p.psink != nullptr;
  // Every wave takes part in every tile's wait, barrier and copies (tile
  // `it` of the flattened (head, query tile) order lives in stage it % NSQ),
  // but computes only the query tiles its keys can see: per head, rows from
  // its first key to its last key's window end.  Three loops per head keep
  // the tile body free of a branch.
  auto sync = [&](int it) {
    // this wave's copies of tile it have landed (the later tiles in flight
    // each add at least LPT newer copies) ...
    if (NSQ == 3 && it + 1 < n_it) wait_vm<LPT>(); else wait_vm<0>();
    lds_barrier();   // ... and everyone's; the stage of tile it-1 is free again
    if (it + NSQ - 1 < n_it) {
      const int b = it % NSQ;
      fetch(f_hg, f_qt, b == 0 ? NSQ - 1 : b - 1);
      advance(f_hg, f_qt);
    }
  };
  int qt_lo = 0, qt_hi = nqt;
  {
    qt_lo = min(nqt, (jw - j0) / RQ);                                   // rows before the first key
    if (W > 0) qt_hi = min(nqt, (jw - j0 + KW - 1 + W - 1) / RQ + 1);   // rows past the last key's window
    if (jw >= L) qt_hi = qt_lo;                                         // no keys
    qt_hi = max(qt_hi, qt_lo);
  }
  int it = 0;
  for (int hg = 0; hg < grp; ++hg) {
    for (int qt = 0; qt < qt_lo; ++qt, ++it) sync(it);
    for (int qt = qt_lo; qt < qt_hi; ++qt, ++it) {
      sync(it);
      const int buf = it % NSQ;
      const int h = kvh * grp + hg;
      const int i0 = j0 + qt * RQ;
      float gk[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) gk[kb] = GATED ? gk_lds[buf][wave][kb * 16 + li] : 0.f;

      // masked pairs give P = dS = 0; the per-element mask runs only on
      // tiles that need it
      const bool need_mask = (i0 < jw + KW - 1) || (W > 0 && i0 + RQ - 1 - jw >= W) || (i0 + RQ > L) ||
                             (jw + KW > L);
      {
        const uint8_t* ql = q_lds[buf];
        const uint8_t* ol = do_lds[buf];
        const float* rowl = row_lds[buf][0];
        const float* dell = row_lds[buf][1];
        // ---- S = Q K^T, dP = dO V^T: C lane (key li, rows rb*16+4g+i) ----
        f32x4 s[KBW][2], dp[KBW][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) {
            s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        {
          // operand reads j = 0 .. NJ-1 (row block j / NR; then Q k-steps,
          // then dO k-steps), issued one chunk of PC reads ahead of their
          // MFMAs (the compiler otherwise waits for each read right away)
          constexpr int NR = KSQ + KSV, NJ = 2 * NR, PC = 2, NC = NJ / PC;
          static_assert(NJ % PC == 0, "chunks");
          bf16x8 a[2][PC];
          auto rd = [&](int j) -> bf16x8 {
            const int rb = j % 2, r = j / 2;   // the two row blocks' chains alternate
            return r < KSQ ? *reinterpret_cast<const bf16x8*>(ql + tile_off<QRB>(rb * 16 + li, 64 * r + 16 * g))
                           : *reinterpret_cast<const bf16x8*>(ol + tile_off<ORB>(rb * 16 + li, 64 * (r - KSQ) + 16 * g));
          };
#pragma unroll
          for (int j = 0; j < PC; ++j) a[0][j] = rd(j);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if (c + 1 < NC) {
#pragma unroll
              for (int j = 0; j < PC; ++j) a[(c + 1) & 1][j] = rd((c + 1) * PC + j);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < PC; ++j) {
              const int jj = c * PC + j, rb = jj % 2, r = jj / 2;
#pragma unroll
              for (int kb = 0; kb < KBW; ++kb) {
                if (r < KSQ) s[kb][rb] = mfma16x16x32(a[c & 1][j], kop[kb][r], s[kb][rb]);
                else dp[kb][rb] = mfma16x16x32(a[c & 1][j], vop[kb][r - KSQ], dp[kb][rb]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- P (masked only on tiles that need it) and dS ----
        f32x4 pv[KBW][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // row term in base 2: gate of the row minus lse
          const f32x4 rowt = *reinterpret_cast<const f32x4*>(rowl + rb * 16 + 4 * g);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pv[kb][rb][i] = fast_exp2(__builtin_fmaf(s[kb][rb][i], p.scale_log2, rowt[i] - gk[kb]));
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
          if constexpr (STORE) {
            if (has_psink) {
              // sink gradient, key side: sum over rows of psink_i P_ij dP_ij
              const float* psl = row_lds[buf][STORE ? 2 : 0];
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) {
                const f32x4 ps4 = *reinterpret_cast<const f32x4*>(psl + rb * 16 + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) sinkcol[kb] = __builtin_fmaf(pv[kb][rb][i] * ps4[i], dp[kb][rb][i], sinkcol[kb]);
              }
            }
            // dS tile of (head h, row tile i0 / 32, this wave's key block)
            const int rt = i0 / kDsRows;
            const int slot = jw / kDsKeys - ds_kb_lo(rt, W);
            if (slot >= 0 && slot < p.ds_nslot) {   // always, for the tiles a wave computes
              const long t = ds_tile(h, ds_grt(seq0, n, rt), slot, p.ds_nrt, p.ds_nslot);
              uint8_t* tb = reinterpret_cast<uint8_t*>(p.ds) + t * kDsTileBytes;
              *reinterpret_cast<bf16x4*>(tb + ds_off(li, 4 * g)) = to_bf16x4(dsv[0]);
              *reinterpret_cast<bf16x4*>(tb + ds_off(li, 16 + 4 * g)) = to_bf16x4(dsv[1]);
              if constexpr (GATED) {
                // fp32 row sums over the block's 16 keys (lanes li): a
                // reduce-scatter over lane bits 3, 2, 1, then a pair sum;
                // lane li ends with the row 16 b3 + 4 g + 2 b2 + b1
                float a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float keep = b3 ? dsv[1][j] : dsv[0][j], send = b3 ? dsv[0][j] : dsv[1][j];
                  a[j] = keep + dpp_f32<0x140>(send);   // row_mirror: partner 15 - li
                }
                float c[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                  const float keep = b2 ? a[2 + j] : a[j], send = b2 ? a[j] : a[2 + j];
                  c[j] = keep + dpp_f32<0x141>(send);   // row_half_mirror: partner flips bits 2..0
                }
                const float keep = b1 ? c[1] : c[0], send = b1 ? c[0] : c[1];
                float r = keep + dpp_f32<0x4e>(send);   // quad_perm [2,3,0,1]: partner li ^ 2
                r += dpp_f32<0xb1>(r);                   // quad_perm [1,0,3,2]: partner li ^ 1
                if ((li & 1) == 0)
                  p.ds_rows[t * kDsRows + 16 * b3 + 4 * g + 2 * b2 + b1] = r;
              }
            }
          }
        }
        // ---- dV^T += dO^T P, dK^T += Q^T dS (32 rows per MFMA) ----
        const int mm = li >> 2, c4 = li & 3;
        const int r0 = 4 * g + mm, r1 = r0 + 16;
#pragma unroll
        for (int db = 0; db < DBV; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(ol + tile_off<ORB>(r0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(ol + tile_off<ORB>(r1, b))));
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) dv_acc[kb][db] = mfma16x16x32(a, pop[kb], dv_acc[kb][db]);
        }
#pragma unroll
        for (int db = 0; db < DBQ; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(ql + tile_off<QRB>(r0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(ql + tile_off<QRB>(r1, b))));
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) dk_acc[kb][db] = mfma16x16x32(a, dsop[kb], dk_acc[kb][db]);
        }
      }
    }
    for (int qt = qt_hi; qt < nqt; ++qt, ++it) sync(it);
    if (GATED) {
      const int h = kvh * grp + hg;
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const float cs = xgroup_sum(colsum[kb]);
        const int key = jw + kb * 16 + li;
        if (g == 0 && key < L) p.dGcol[(long)h * p.T + seq0 + key] = cs;   // head-major
        colsum[kb] = 0.f;
      }
    }
    if (has_psink) {
      const int h = kvh * grp + hg;
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const float sc = xgroup_sum(sinkcol[kb]);
        const int key = jw + kb * 16 + li;
        if (g == 0 && key < L) p.sink_rows[(long)h * p.T + seq0 + key] = sc;   // per key, head-major
        sinkcol[kb] = 0.f;
      }
    }
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
  constexpr int KRB = DQK * 2, VRB = DV * 2;   // bytes per K / V row
  static_assert(KB % 2 == 0, "dQ consumes keys in pairs of 16-key blocks");
  static_assert(BN <= 64, "gate copy is one lane per key");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][BN * VRB];
  __shared__ __attribute__((aligned(16))) float gk_lds[2][4][64];   // one copy per wave

  const int h = xcd_remap(blockIdx.x, p.Hq), n = blockIdx.z;
  const int tile = gridDim.y - 1 - blockIdx.y;
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
    dlt[rb] = ok ? p.delta[(long)h * p.T + seq0 + row] : 0.f;
    gq[rb] = (ok && gated) ? p.G2[(long)h * p.T + seq0 + min(row, L - 1)] : 0.f;
    rowsum[rb] = 0.f;
    pdp[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) dq_acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int kv_lo = W > 0 ? max(0, i0 - W + 1) : 0;
  const int kv_hi = min(L, i0 + BM);
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + ((long)seq0 * p.Hkv + kvh) * VRB;
  const int kstride = p.Hkv * KRB, vstride = p.Hkv * VRB;

  // K/V tiles (and each wave's copy of the key gate terms) go global -> LDS
  // by direct copies into a two-stage ring of swizzled tiles, one tile
  // ahead of the math (as in the forward kernel): wave w copies the 1 KB
  // blocks w, w+4, ... of each tile; rows past the end re-read the last row
  // (finite; masked).
  constexpr int KPW = BN * KRB / 4096, VPW = BN * VRB / 4096;
  static_assert(KPW * 4096 == BN * KRB && VPW * 4096 == BN * VRB, "tile must split into 4 x k 1 KB blocks");
  int krow[KPW], koff[KPW], vrow[VPW], voff[VPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    krow[j] = o / KRB;
    koff[j] = krow[j] * kstride + ((((o % KRB) >> 4) ^ tile_swz<KRB>(krow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    vrow[j] = o / VRB;
    voff[j] = vrow[j] * vstride + ((((o % VRB) >> 4) ^ tile_swz<VRB>(vrow[j])) << 4);
  }
  const float* g2base = GATED ? p.G2 + (long)h * p.T + seq0 : nullptr;
  auto fetch = [&](int st, int j0) {
    const bool tail = j0 + BN > L;               // uniform: only the last tile clamps
    const uint8_t* kb = kbase + (long)j0 * kstride;
    const uint8_t* vb = vbase + (long)j0 * vstride;
    const uint32_t kl = lds_addr(k_lds[st]), vl = lds_addr(v_lds[st]);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int over = tail ? max(0, j0 + krow[j] - (L - 1)) : 0;
      dma16(kb, (uint32_t)(koff[j] - over * kstride), kl + (wave + 4 * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int over = tail ? max(0, j0 + vrow[j] - (L - 1)) : 0;
      dma16(vb, (uint32_t)(voff[j] - over * vstride), vl + (wave + 4 * j) * 1024);
    }
    if constexpr (GATED)
      dma4(g2base, (uint32_t)(min(j0 + lane, L - 1) * 4), lds_addr(&gk_lds[st][wave][0]));
  };

  if (t_begin < t_end) fetch(0, t_begin * BN);

  // Every wave takes part in every tile's wait, barrier and copies, but
  // computes only the key tiles its rows can see (from the first row's
  // window start to the last row); three loops keep the tile body free of
  // a branch.  Inside that range, masked pairs contribute zeros; rows past
  // the end are masked too, their lse is not defined.
  auto sync = [&](int t) {
    wait_vm<0>();     // this wave's copies of tile t have landed
    lds_barrier();    // ... and everyone's; the other stage is free again
    if (t + 1 < t_end) fetch(((t - t_begin) & 1) ^ 1, t * BN + BN);
  };
  int tw_lo = t_begin, tw_hi = t_end;
  {
    if (W > 0 && r0 - W + 1 > 0) tw_lo = max(t_begin, (r0 - W + 1) / BN);
    tw_hi = r_last >= r0 ? min(t_end, r_last / BN + 1) : t_begin;
    tw_lo = min(tw_lo, tw_hi);
  }
  for (int t = t_begin; t < tw_lo; ++t) sync(t);
  for (int t = tw_lo; t < tw_hi; ++t) {
    const int j0 = t * BN;
    const int buf = (t - t_begin) & 1;
    sync(t);
    {
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + RW - 1);
      const uint8_t* kl = k_lds[buf];
      const uint8_t* vl = v_lds[buf];
      f32x4 s[KB][RBW], dp[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      {
        // operand reads j = 0 .. NJ-1 (key block j / NR; then K k-steps,
        // then V k-steps), issued one chunk of PC reads ahead of their MFMAs
        constexpr int NR = KSQ + KSV, NJ = KB * NR, PC = 2, NC = NJ / PC;
        static_assert(NJ % PC == 0, "chunks");
        bf16x8 a[2][PC];
        auto rd = [&](int j) -> bf16x8 {
          const int kb = j / NR, r = j % NR;
          return r < KSQ ? *reinterpret_cast<const bf16x8*>(kl + tile_off<KRB>(kb * 16 + li, 64 * r + 16 * g))
                         : *reinterpret_cast<const bf16x8*>(vl + tile_off<VRB>(kb * 16 + li, 64 * (r - KSQ) + 16 * g));
        };
#pragma unroll
        for (int j = 0; j < PC; ++j) a[0][j] = rd(j);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c + 1 < NC) {
#pragma unroll
            for (int j = 0; j < PC; ++j) a[(c + 1) & 1][j] = rd((c + 1) * PC + j);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < PC; ++j) {
            const int jj = c * PC + j, kb = jj / NR, r = jj % NR;
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
              if (r < KSQ) s[kb][rb] = mfma16x16x32(a[c & 1][j], qop[rb][r], s[kb][rb]);
              else dp[kb][rb] = mfma16x16x32(a[c & 1][j], doop[rb][r - KSQ], dp[kb][rb]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- P (masked only on tiles that need it), dS, row sums ----
      f32x4 pv[KB][RBW];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 gk = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) gk = *reinterpret_cast<const f32x4*>(&gk_lds[buf][wave][kb * 16 + 4 * g]);
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
        const int kr0 = kp * 32 + 4 * g + mm, kr1 = kr0 + 16;
#pragma unroll
        for (int db = 0; db < DBQ; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(kl + tile_off<KRB>(kr0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(kl + tile_off<KRB>(kr1, b))));
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
            dq_acc[rb][db] = mfma16x16x32(a, concat(dsb[2 * kp][rb], dsb[2 * kp + 1][rb]), dq_acc[rb][db]);
        }
      }
    }
  }
  for (int t = tw_hi; t < t_end; ++t) sync(t);

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
      const long hm = (long)h * p.T + seq0 + row;   // head-major
      if (gated) p.dGrow[hm] = rs;
      if (p.sink) p.sink_rows[hm] = fast_exp2(sink2 - lse2[rb]) * sp;
    }
  }
}

template <int DQK, int DV>
struct BwdTiles {
  // dQ pass: 32 rows per wave and 64-key tiles while Q, dO and the K/V ring
  // stay small; 16 rows and 32-key tiles for the larger heads (registers and
  // the 64 KB-per-stage LDS ring).
  static constexpr bool small = DQK + DV <= 256;
  static constexpr int KW = kBwdKwSmall;
  static constexpr int RW = small ? kBwdRwSmall : 16;
  static constexpr int BN = small ? 64 : 32;
};

template <int DQK, int DV>
hipError_t launch_bwd_two_pass_t(const BwdParams& p, hipStream_t st) {
  constexpr int KW = BwdTiles<DQK, DV>::KW, RW = BwdTiles<DQK, DV>::RW, BN = BwdTiles<DQK, DV>::BN;
  hipError_t e;
  if constexpr (DQK == 256 && DV >= 256) {
    e = launch_dkdv_large(p, DQK, DV, st);   // bwd_large.hip
  } else {
    const int ktiles = (p.max_seqlen + 4 * KW - 1) / (4 * KW);
    const dim3 gk(p.Hkv, ktiles, p.num_seqs);   // sequence-major: a sequence's tiles share L2
    if (p.ds != nullptr) {
      if (p.G2) bwd_dkdv_kernel<DQK, DV, KW, true, true><<<gk, 256, 0, st>>>(p);
      else bwd_dkdv_kernel<DQK, DV, KW, false, true><<<gk, 256, 0, st>>>(p);
    } else {
      if (p.G2) bwd_dkdv_kernel<DQK, DV, KW, true, false><<<gk, 256, 0, st>>>(p);
      else bwd_dkdv_kernel<DQK, DV, KW, false, false><<<gk, 256, 0, st>>>(p);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (p.ds != nullptr) {
    // dQ from the stored dS: 128 rows per workgroup
    const dim3 gq(p.Hq, (p.max_seqlen + 4 * kDsRows - 1) / (4 * kDsRows), p.num_seqs);
    bwd_dq_ds_kernel<DQK><<<gq, 256, 0, st>>>(p);
    e = hipGetLastError();
  } else if constexpr (DQK == 256 && DV >= 256) {
    e = launch_dq_large(p, DQK, DV, st);   // bwd_large.hip
  } else {
    const int qtiles = (p.max_seqlen + 4 * RW - 1) / (4 * RW);
    const dim3 gq(p.Hq, qtiles, p.num_seqs);
    if (p.G2) bwd_dq_kernel<DQK, DV, RW, BN, true><<<gq, 256, 0, st>>>(p);
    else bwd_dq_kernel<DQK, DV, RW, BN, false><<<gq, 256, 0, st>>>(p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return p.sink ? launch_sink_reduce(p, st) : hipSuccess;
}

// One entry per query/key head dim (bwd2.hip, bwd2_qk128.hip, bwd2_qk256.hip).
template <int DQK>
hipError_t launch_bwd_two_pass_qk(const BwdParams& p, int dv, hipStream_t st) {
  switch (dv) {
    case 64: return launch_bwd_two_pass_t<DQK, 64>(p, st);
    case 128: return launch_bwd_two_pass_t<DQK, 128>(p, st);
    case 256: return launch_bwd_two_pass_t<DQK, 256>(p, st);
    case 512: return launch_bwd_two_pass_t<DQK, 512>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
