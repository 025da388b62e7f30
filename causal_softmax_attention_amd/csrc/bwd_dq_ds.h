// dQ pass of the two-pass backward from a stored dS (layout in bwd_ds.h), for
// gfx950: dq_i = scale * sum_j dS_ij k_j, and for the gate the row sums
// sum_j dS_ij from the fp32 per-block partials the dK/dV pass stored.
//
// One workgroup of four wavefronts per (query head, 128 query rows,
// sequence); wavefront w owns the 32 rows of one dS row tile.  K tiles of BN
// keys (64, or 32 for d_qk 256) and each wave's dS tiles of those keys reach
// LDS by direct copies into a two-stage ring, one tile ahead; dQ^T
// accumulates in registers from K^T (ds_read_b64_tr_b16) times dS^T (the
// stored key-major tiles, read transposed).  Blocks outside a row tile's
// band were never written: their operands are zero.
#pragma once
#include "bwd_ds.h"
#include "common.h"
#include "kernels.h"

namespace attn {

template <int DQK>
__global__ __launch_bounds__(256) void bwd_dq_ds_kernel(BwdParams p) {
  constexpr int RW = kDsRows;                // rows per wave
  constexpr int BN = DQK <= 128 ? 64 : 32;   // keys per K tile
  constexpr int NB = BN / kDsKeys;           // dS key blocks per tile
  constexpr int DBQ = DQK / 16;
  constexpr int KRB = DQK * 2;               // bytes per K row
  constexpr int KPW = BN * KRB / 4096;       // 1 KB K copy blocks per wave
  static_assert(KPW * 4096 == BN * KRB && NB % 2 == 0, "tile split");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t ds_lds[2][4][NB][kDsTileBytes];

  const int h = xcd_remap(blockIdx.x, p.Hq), n = blockIdx.z;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int i0 = (gridDim.y - 1 - blockIdx.y) * 4 * RW;   // longest rows first
  if (i0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int kvh = h / grp;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
  const int rt = i0 / RW + wave;             // this wave's row tile
  const bool rows_ok = rt * RW < L;          // wave-uniform
  const int kb_lo = ds_kb_lo(rt, W);
  const int kb_hi = rows_ok ? ds_kb_hi(rt, L) : kb_lo - 1;   // empty band past the end
  const long grt = ds_grt(seq0, n, rt);
  const long tbase = ds_tile(h, grt, 0, p.ds_nrt, p.ds_nslot);   // slot 0 of the row tile

  // key tiles the workgroup streams: the union of its waves' bands
  const int rt_last = min(i0 / RW + 3, (L - 1) / RW);
  const int t_begin = ds_kb_lo(i0 / RW, W) * kDsKeys / BN;
  const int t_end = (ds_kb_hi(rt_last, L) * kDsKeys) / BN + 1;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + ((long)seq0 * p.Hkv + kvh) * KRB;
  const int kstride = p.Hkv * KRB;
  int krow[KPW], koff[KPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int o = (wave + 4 * j) * 1024 + lane * 16;
    krow[j] = o / KRB;
    koff[j] = krow[j] * kstride + ((((o % KRB) >> 4) ^ tile_swz<KRB>(krow[j])) << 4);
  }
  const uint8_t* dsb = reinterpret_cast<const uint8_t*>(p.ds);
  auto fetch = [&](int st, int t) {
    const int j0 = t * BN;
    const bool tail = j0 + BN > L;           // uniform: only the last tile clamps
    const uint8_t* kb = kbase + (long)j0 * kstride;
    const uint32_t kl = lds_addr(k_lds[st]);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int over = tail ? max(0, j0 + krow[j] - (L - 1)) : 0;   // rows past the end re-read the last
      dma16(kb, (uint32_t)(koff[j] - over * kstride), kl + (wave + 4 * j) * 1024);
    }
    // this wave's dS tiles of the key blocks in its band (1 KB each, linear)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int kb2 = t * NB + b;
      if (kb2 >= kb_lo && kb2 <= kb_hi)
        dma16(sgpr_ptr(dsb + (tbase + (kb2 - kb_lo)) * kDsTileBytes), (uint32_t)(lane * 16),
              lds_addr(ds_lds[st][wave][b]));
    }
  };

  f32x4 dq_acc[2][DBQ];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DBQ; ++db) dq_acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (t_begin < t_end) fetch(0, t_begin);
  auto sync = [&](int t) {
    wait_vm<0>();     // this wave's copies of tile t have landed
    lds_barrier();    // ... and everyone's; the other stage is free again
    if (t + 1 < t_end) fetch(((t - t_begin) & 1) ^ 1, t + 1);
  };
  // tiles this wave computes: those holding a block of its band
  const int tw_lo = min(max(t_begin, kb_lo * kDsKeys / BN), t_end);
  const int tw_hi = kb_hi < kb_lo ? tw_lo : max(tw_lo, min(t_end, kb_hi * kDsKeys / BN + 1));
  // transposed-read offsets: K^T (keys 4 g + mm and + 16 of a 32-key pair,
  // columns 32 db + 8 c4) and dS^T (key 4 g + mm, rows 16 rb + 4 c4)
  const int mm = li >> 2, c4 = li & 3;
  for (int t = t_begin; t < tw_lo; ++t) sync(t);
  for (int t = tw_lo; t < tw_hi; ++t) {
    sync(t);
    const int buf = (t - t_begin) & 1;
    const uint8_t* kl = k_lds[buf];
#pragma unroll
    for (int kp = 0; kp < NB / 2; ++kp) {
      bf16x8 bop[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        bf16x4 half[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int b = 2 * kp + e, kb2 = t * NB + b;
          const bool ok = kb2 >= kb_lo && kb2 <= kb_hi;   // wave-uniform
          const bf16x4 x = lds_read_tr16(reinterpret_cast<const bf16*>(ds_lds[buf][wave][b] +
                                                                       ds_off(4 * g + mm, 16 * rb + 4 * c4)));
          half[e] = ok ? x : bf16x4{};
        }
        bop[rb] = concat(half[0], half[1]);
      }
      const int kr0 = kp * 32 + 4 * g + mm, kr1 = kr0 + 16;
#pragma unroll
      for (int db = 0; db < DBQ; ++db) {
        const int b = 32 * db + 8 * c4;
        const bf16x8 a = concat(lds_read_tr16(reinterpret_cast<const bf16*>(kl + tile_off<KRB>(kr0, b))),
                                lds_read_tr16(reinterpret_cast<const bf16*>(kl + tile_off<KRB>(kr1, b))));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) dq_acc[rb][db] = mfma16x16x32(a, bop[rb], dq_acc[rb][db]);
      }
    }
  }
  for (int t = tw_hi; t < t_end; ++t) sync(t);

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = rt * RW + rb * 16 + li;
    // gate: row sums of dS from the per-block partials, lane group g adding
    // blocks g, g + 4, ... in order, then the four groups
    float rs = 0.f;
    if (p.dGrow != nullptr) {
      for (int b = g; b <= kb_hi - kb_lo; b += 4) rs += p.ds_rows[(tbase + b) * kDsRows + rb * 16 + li];
      rs = xgroup_sum(rs);
    }
    if (!rows_ok || row >= L) continue;
    const long ri = (long)(seq0 + row) * p.Hq + h;
    bf16* dqp = reinterpret_cast<bf16*>(p.dq) + ri * DQK + 4 * g;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) *reinterpret_cast<bf16x4*>(dqp + db * 16) = to_bf16x4(dq_acc[rb][db] * p.scale);
    if (g == 0 && p.dGrow != nullptr) p.dGrow[(long)h * p.T + seq0 + row] = rs;
  }
}

}  // namespace attn
