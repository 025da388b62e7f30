// Fused-dQ backward for gfx950: dQ accumulated in the dK/dV pass through
// fp32 atomics, so each score and dP tile is computed once.
//
// Method (fla issue #1322, comment of Oct 5): dQ fused into the dK/dV pass,
// its partials added into a zero-initialised fp32 buffer and converted to
// the input dtype afterwards; the gate and sink gradients as fp32 partial
// sums (comment of Oct 3: the sink gradient summed directly from
// P * (dO V^T) with the sink probability).
//
// gfx950 mapping.  One workgroup of 8 wavefronts per (128-key block, KV
// head, sequence) (4 wavefronts and 64 keys for value heads of 256 and
// more); each wave keeps K and V of its 16 keys in registers (the
// B operands of S = Q K^T and dP = dO V^T) and its dK^T, dV^T accumulators,
// and walks the 32-row query tiles of the group's heads that its keys see.
// Q and dO tiles (with the per-row terms and the keys' gate terms) arrive
// by direct global->LDS copies into a two-stage ring of swizzled tiles.  Per
// tile each wave writes its dS (bf16, key-major, chunk-swizzled) to LDS;
// after a barrier every wave multiplies the whole 32-row dS tile by K for
// its slice of d_qk (K^T fragments held in registers from the start) and
// adds the result to dQ with one fp32 atomic per element: the partials of
// the block's keys are summed in registers before they reach memory (measured on
// one MI355X: device-scope fp32 atomics run at about 330 G elements/s, so
// the atomic traffic, not the MFMA work, sets the pace).  Row sums of dS
// (gate gradient) are reduced across the waves in LDS, one atomic per row.
#pragma once
#include "common.h"
#include "kernels.h"

namespace attn {

// Wavefronts per workgroup: 8 (128 keys), or 4 (64 keys) for value heads of
// 256 and more, whose dV accumulators need the registers of a whole SIMD.
template <int DV>
constexpr int fused_waves() { return DV >= 256 ? 4 : 8; }

template <int DQK, int DV, bool GATED>
__global__ __launch_bounds__(64 * fused_waves<DV>()) void bwd_fused_kernel(BwdParams p) {
  constexpr int NW = fused_waves<DV>(), KW = 16;
  constexpr int BNW = NW * KW;        // keys per workgroup
  constexpr int RQ = 32;              // query rows per tile
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int DBQ = DQK / 16, DBV = DV / 16;
  constexpr int QRB = DQK * 2, ORB = DV * 2;   // bytes per Q / dO row
  constexpr int QBLK = RQ * QRB / 1024, OBLK = RQ * ORB / 1024;   // 1 KB copy blocks
  constexpr int QPW = (QBLK + NW - 1) / NW, OPW = (OBLK + NW - 1) / NW;
  constexpr int NDQ = DQK / 16;       // 16-column blocks of dQ
  constexpr int NIT = NDQ * 2 / NW;   // dQ items (column block, 16-row block) per wave
  constexpr int NCB = NDQ >= NW ? NDQ / NW : 1;   // distinct column blocks per wave
  constexpr int DSRB = RQ * 2;        // key-major dS rows: 64 bytes
  static_assert(NDQ * 2 % NW == 0 && NIT >= 1, "dQ work split");
  static_assert(DQK <= 128, "fused path: d_qk <= 128");
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds[2][RQ * QRB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds[2][RQ * ORB];
  __shared__ __attribute__((aligned(16))) uint8_t ds_lds[BNW * DSRB];
  __shared__ __attribute__((aligned(16))) float row_lds[2][3][64];      // row term, delta, lse
  __shared__ __attribute__((aligned(16))) float gk_lds[2][NW][64];      // per wave: its keys' gate terms
  __shared__ __attribute__((aligned(16))) float rs_lds[NW][RQ];         // dS row sums per wave

  const int kvh = blockIdx.x, n = blockIdx.z, ktile = blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int j0 = ktile * BNW;
  if (j0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
  const int jw = j0 + wave * KW;
  const int key = jw + li;            // this lane's key (S / dP columns)

  bf16x8 kop[KSQ], vop[KSV];
  {
    const bool ok = key < L;
    const long kr = (long)(seq0 + min(key, L - 1)) * p.Hkv + kvh;
    const bf16* kp = reinterpret_cast<const bf16*>(p.k) + kr * DQK + 8 * g;
    const bf16* vp = reinterpret_cast<const bf16*>(p.v) + kr * DV + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) kop[ks] = ok ? *reinterpret_cast<const bf16x8*>(kp + 32 * ks) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) vop[ks] = ok ? *reinterpret_cast<const bf16x8*>(vp + 32 * ks) : bf16x8{};
  }
  // dQ items of this wave: x = wave + NW t (t < NIT), column block x % NDQ,
  // row block x / NDQ; item t uses column block (wave + NW (t % NCB)) % NDQ.
  // K^T fragments of the dQ product per column block (B operand: lane column
  // 16 cb + l % 16, keys 32 ks + 8 g .. + 7 of the block)
  bf16x8 ktf[NCB][BNW / 32];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int cb = (wave + NW * c) % NDQ;
    const bf16* kb = reinterpret_cast<const bf16*>(p.k) + (long)kvh * DQK + 16 * cb + li;
#pragma unroll
    for (int ks = 0; ks < BNW / 32; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = j0 + 32 * ks + 8 * g + e;
        ktf[c][ks][e] = kk < L ? kb[(long)(seq0 + kk) * p.Hkv * DQK] : (bf16)0.f;
      }
  }
  f32x4 dk_acc[DBQ], dv_acc[DBV];
#pragma unroll
  for (int db = 0; db < DBQ; ++db) dk_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < DBV; ++db) dv_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int i_end = W > 0 ? min(L, j0 + BNW - 1 + W) : L;
  const int nqt = (i_end - j0 + RQ - 1) / RQ;
  const int n_it = grp * nqt;

  const int qstride = p.Hq * QRB, ostride = p.Hq * ORB;
  int qrow[QPW], qoff[QPW], orow[OPW], ooff[OPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    qrow[j] = o / QRB;
    qoff[j] = qrow[j] * qstride + ((((o % QRB) >> 4) ^ tile_swz<QRB>(qrow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < OPW; ++j) {
    const int o = (wave + NW * j) * 1024 + lane * 16;
    orow[j] = o / ORB;
    ooff[j] = orow[j] * ostride + ((((o % ORB) >> 4) ^ tile_swz<ORB>(orow[j])) << 4);
  }
  auto fetch = [&](int hg, int qt, int st) {
    const int hh = kvh * grp + hg;
    const int i0 = j0 + qt * RQ;
    const bool tail = i0 + RQ > L;
    const long r0 = (long)(seq0 + i0) * p.Hq + hh;
    const uint8_t* qb = sgpr_ptr(reinterpret_cast<const uint8_t*>(p.q) + r0 * QRB);
    const uint8_t* ob = sgpr_ptr(reinterpret_cast<const uint8_t*>(p.dO) + r0 * ORB);
    const uint32_t ql = lds_addr(q_lds[st]), ol = lds_addr(do_lds[st]);
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      if (QBLK % NW != 0 && wave + NW * j >= QBLK) break;   // uniform
      const int over = tail ? max(0, i0 + qrow[j] - (L - 1)) : 0;   // rows past the end re-read the last
      dma16(qb, (uint32_t)(qoff[j] - over * qstride), ql + (wave + NW * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < OPW; ++j) {
      if (OBLK % NW != 0 && wave + NW * j >= OBLK) break;
      const int over = tail ? max(0, i0 + orow[j] - (L - 1)) : 0;
      dma16(ob, (uint32_t)(ooff[j] - over * ostride), ol + (wave + NW * j) * 1024);
    }
    if (wave == 0) {
      // per-row terms, lane l -> row min(i0 + l % RQ, L - 1)
      const int rr = min(i0 + (lane % RQ), L - 1) - i0;
      const long hr = (long)hh * p.T + seq0 + i0;
      dma4(sgpr_ptr(p.rowt + hr), (uint32_t)(rr * 4), lds_addr(&row_lds[st][0][0]));
      dma4(sgpr_ptr(p.delta + hr), (uint32_t)(rr * 4), lds_addr(&row_lds[st][1][0]));
      if (p.sink)
        dma4(sgpr_ptr(p.lse + (long)(seq0 + i0) * p.Hq + hh), (uint32_t)(rr * p.Hq * 4), lds_addr(&row_lds[st][2][0]));
    }
    if constexpr (GATED) {
      const uint32_t ko = (uint32_t)(min(jw + (lane % KW), L - 1) * 4);
      dma4(sgpr_ptr(p.G2 + (long)hh * p.T + seq0), ko, lds_addr(&gk_lds[st][wave][0]));
    }
  };

#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks) asm volatile("" :: "v"(kop[ks]));
#pragma unroll
  for (int ks = 0; ks < KSV; ++ks) asm volatile("" :: "v"(vop[ks]));
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int ks = 0; ks < BNW / 32; ++ks) asm volatile("" :: "v"(ktf[c][ks]));

  // dS tile, key-major: local key kl (row of 64 bytes), query rows as
  // columns; chunk c of key kl at c ^ ds_swz(kl), so that the 8 keys of a
  // transposed read (kl and kl + 8 share banks) use both 32-byte halves
  auto ds_swz = [](int kl) { return ((kl >> 3) & 1) << 1; };
  const int kl_w = wave * KW + li;
  uint32_t ds_wr[2];   // rows rb * 16 + 4 g .. + 3 of key kl_w
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
    ds_wr[rb] = (uint32_t)(kl_w * DSRB + (((2 * rb + (g >> 1)) ^ ds_swz(kl_w)) << 4) + 8 * (g & 1));
  // dQ A operand (transposed reads): keys 32 ks + 8 g + 4 r + (l % 16) / 4,
  // rows rb * 16 + 4 (l % 4) .. + 3
  const int tq = lane & 15;
  uint32_t ds_rd[NIT][2];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int rb = (wave + NW * it) / NDQ;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int kl = 8 * g + 4 * r + (tq >> 2);   // + 32 ks (keeps ds_swz)
      ds_rd[it][r] = (uint32_t)(kl * DSRB + (((2 * rb + ((tq & 3) >> 1)) ^ ds_swz(kl)) << 4) + 8 * (tq & 1));
    }
  }

  int f_hg = 0, f_qt = 0;
  fetch(0, 0, 0);
  if (++f_qt == nqt) { f_qt = 0; ++f_hg; }
  float colsum = 0.f, sink_part = 0.f;
  // this wave's query tiles per head: from its first key's row to its last
  // key's window end
  int qt_lo = min(nqt, (jw - j0) / RQ);
  int qt_hi = nqt;
  if (W > 0) qt_hi = min(nqt, (jw - j0 + KW - 1 + W - 1) / RQ + 1);
  if (jw >= L) qt_hi = qt_lo;
  qt_hi = max(qt_hi, qt_lo);

  int it = 0;
  for (int hg = 0; hg < grp; ++hg) {
    const int h = kvh * grp + hg;
    const float sink2 = p.sink ? p.sink[h] * kLog2e : 0.f;
    for (int qt = 0; qt < nqt; ++qt, ++it) {
      const int st = it & 1;
      wait_vm<0>();
      lds_barrier();   // tile it landed; the previous tile's LDS (stage, dS, row sums) is free
      if (it + 1 < n_it) {
        fetch(f_hg, f_qt, st ^ 1);
        if (++f_qt == nqt) { f_qt = 0; ++f_hg; }
      }
      const int i0 = j0 + qt * RQ;
      if (qt >= qt_lo && qt < qt_hi) {
        const uint8_t* ql = q_lds[st];
        const uint8_t* ol = do_lds[st];
        const float* rowl = row_lds[st][0];
        const float* dell = row_lds[st][1];
        const float gk = GATED ? gk_lds[st][wave][li] : 0.f;
        const bool need_mask = (i0 < jw + KW - 1) || (W > 0 && i0 + RQ - 1 - jw >= W) || (i0 + RQ > L) ||
                               (jw + KW > L);
        // ---- S = Q K^T, dP = dO V^T: C lane (key li, rows rb*16+4g+i) ----
        f32x4 s[2], dp[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // the two row blocks' chains alternate
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            s[rb] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(ql + tile_off<QRB>(rb * 16 + li, 64 * ks + 16 * g)),
                                 kop[ks], s[rb]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            dp[rb] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(ol + tile_off<ORB>(rb * 16 + li, 64 * ks + 16 * g)),
                                  vop[ks], dp[rb]);
        // ---- P, dS, partial sums ----
        f32x4 pv[2], dsv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 rowt = *reinterpret_cast<const f32x4*>(rowl + rb * 16 + 4 * g);
          const f32x4 del4 = *reinterpret_cast<const f32x4*>(dell + rb * 16 + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[rb][i] = fast_exp2(__builtin_fmaf(s[rb][i], p.scale_log2, rowt[i] - gk));
          if (need_mask) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = i0 + rb * 16 + 4 * g + i;
              const bool vis = key < L && row < L && key <= row && (W <= 0 || row - key < W);
              pv[rb][i] = vis ? pv[rb][i] : 0.f;
            }
          }
          f32x4 lse2 = {0.f, 0.f, 0.f, 0.f};
          if (p.sink) lse2 = *reinterpret_cast<const f32x4*>(&row_lds[st][2][rb * 16 + 4 * g]) * kLog2e;
          float rsum[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d = pv[rb][i] * (dp[rb][i] - del4[i]);
            dsv[rb][i] = d;
            colsum += d;
            rsum[i] = d;
            if (p.sink) sink_part += fast_exp2(sink2 - lse2[i]) * (pv[rb][i] * dp[rb][i]);
          }
          if constexpr (GATED) {
            // row sums over the wave's 16 keys (the 16 lanes of a group)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v = rsum[i];
              v += __shfl_xor(v, 1);
              v += __shfl_xor(v, 2);
              v += __shfl_xor(v, 4);
              v += __shfl_xor(v, 8);
              if (li == 0) rs_lds[wave][rb * 16 + 4 * g + i] = v;
            }
          }
          *reinterpret_cast<bf16x4*>(ds_lds + ds_wr[rb]) = to_bf16x4(dsv[rb]);
        }
        // ---- dV^T += dO^T P, dK^T += Q^T dS (32 rows per MFMA) ----
        const bf16x8 pop = concat(to_bf16x4(pv[0]), to_bf16x4(pv[1]));
        const bf16x8 dsop = concat(to_bf16x4(dsv[0]), to_bf16x4(dsv[1]));
        const int mm = li >> 2, c4 = li & 3;
        const int r0 = 4 * g + mm, r1 = r0 + 16;
#pragma unroll
        for (int db = 0; db < DBV; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(ol + tile_off<ORB>(r0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(ol + tile_off<ORB>(r1, b))));
          dv_acc[db] = mfma16x16x32(a, pop, dv_acc[db]);
        }
#pragma unroll
        for (int db = 0; db < DBQ; ++db) {
          const int b = 32 * db + 8 * c4;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(ql + tile_off<QRB>(r0, b))),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(ql + tile_off<QRB>(r1, b))));
          dk_acc[db] = mfma16x16x32(a, dsop, dk_acc[db]);
        }
      } else {
        // no visible pair for this wave's keys: zero dS and row sums
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) *reinterpret_cast<bf16x4*>(ds_lds + ds_wr[rb]) = bf16x4{};
        if (GATED && li == 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) rs_lds[wave][rb * 16 + 4 * g + i] = 0.f;
        }
      }
      lds_barrier();   // the tile's dS (and row sums) from every wave

      // ---- dQ[rows][16 cb ..] += dS K over the 128 keys; one atomic per element ----
#pragma unroll
      for (int t = 0; t < NIT; ++t) {
        const int rb = (wave + NW * t) / NDQ;
        const int cb = (wave + NW * (t % NCB)) % NDQ;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < BNW / 32; ++ks) {
          const uint8_t* b = ds_lds + ks * 32 * DSRB;
          const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(b + ds_rd[t][0])),
                                  lds_read_tr16(reinterpret_cast<const bf16*>(b + ds_rd[t][1])));
          c = mfma16x16x32(a, ktf[t % NCB][ks], c);
        }
        // C lane: column 16 cb + li, rows rb*16 + 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = i0 + rb * 16 + 4 * g + i;
          if (row < L) atomicAdd(p.dq_acc + ((long)(seq0 + row) * p.Hq + h) * DQK + 16 * cb + li, c[i] * p.scale);
        }
      }
      if constexpr (GATED) {
        if (wave == 0 && lane < RQ) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) v += rs_lds[w][lane];
          const int row = i0 + lane;
          if (row < L) atomicAdd(p.dG + (long)(seq0 + row) * p.Hq + h, v);
        }
      }
    }
    // ---- per-head partial sums: sink gradient, gate column sums ----
    if (p.sink) {
      float v = sink_part;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && v != 0.f) atomicAdd(p.dsink_acc + h, -v);
      sink_part = 0.f;
    }
    if constexpr (GATED) {
      const float cs = xgroup_sum(colsum);
      if (g == 0 && key < L) atomicAdd(p.dG + (long)(seq0 + key) * p.Hq + h, -cs);
      colsum = 0.f;
    }
  }

  // ---- dK = scale * dK^T acc, dV (lane: key li, columns db*16+4g+i) ----
  if (key < L) {
    bf16* dkp = reinterpret_cast<bf16*>(p.dk) + ((long)(seq0 + key) * p.Hkv + kvh) * DQK + 4 * g;
    bf16* dvp = reinterpret_cast<bf16*>(p.dv) + ((long)(seq0 + key) * p.Hkv + kvh) * DV + 4 * g;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) *reinterpret_cast<bf16x4*>(dkp + db * 16) = to_bf16x4(dk_acc[db] * p.scale);
#pragma unroll
    for (int db = 0; db < DBV; ++db) *reinterpret_cast<bf16x4*>(dvp + db * 16) = to_bf16x4(dv_acc[db]);
  }
}

template <int DQK, int DV>
hipError_t launch_fused_kernel(const BwdParams& p, hipStream_t st) {
  constexpr int NW = fused_waves<DV>();
  const dim3 grid(p.Hkv, (p.max_seqlen + 16 * NW - 1) / (16 * NW), p.num_seqs);
  if (p.G2) bwd_fused_kernel<DQK, DV, true><<<grid, 64 * NW, 0, st>>>(p);
  else bwd_fused_kernel<DQK, DV, false><<<grid, 64 * NW, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace attn
