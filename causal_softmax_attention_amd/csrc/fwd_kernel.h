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
//  * K and V tiles of BN keys are staged in LDS with their 16-byte chunks
//    permuted per row (tile_swz: conflict-free for the MFMA-row and the
//    transposed reads); V^T operands come from ds_read_b64_tr_b16, so P
//    leaves the score registers straight into the PV MFMA with no shuffle.
//  * Online softmax in base 2: scores are scaled by softmax_scale*log2(e)
//    and the gate prefix is stored pre-multiplied by log2(e); the running
//    max starts at the sink logit with l = 1.  Masking is applied only on
//    tiles that cross the diagonal, the window edge or the sequence end.
#pragma once
#include "common.h"
#include "kernels.h"

namespace attn {

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
// Row max of a tile held as sc[kb][rb][i] (keys kb*16 + 4g + i), and a sum
// of per-block partials, both as trees (independent steps instead of one
// dependent chain per row).  The summation order is fixed.
template <int KB, int RBW>
__device__ __forceinline__ float tile_row_max(const f32x4 (&sc)[KB][RBW], int rb) {
  float m[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    m[kb] = fmaxf(fmaxf(fmaxf(sc[kb][rb][0], sc[kb][rb][1]), sc[kb][rb][2]), sc[kb][rb][3]);
#pragma unroll
  for (int w = 1; w < KB; w *= 2)
#pragma unroll
    for (int kb = 0; kb + w < KB; kb += 2 * w) m[kb] = fmaxf(m[kb], m[kb + w]);
  return m[0];
}
template <int N>
__device__ __forceinline__ float tree_sum(float (&v)[N]) {
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int i = 0; i + w < N; i += 2 * w) v[i] += v[i + w];
  return v[0];
}

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2);
// map block x so that the query heads of one KV group land on one XCD.
__device__ __forceinline__ int xcd_head(int x, int Hq) {
  if (Hq % 8 != 0) return x;
  return (x % 8) * (Hq / 8) + x / 8;
}

template <int DQK, int DV, int RW, int BN, int NST, bool GATED, int NWV>
__global__ __launch_bounds__(64 * NWV) void fwd_kernel(FwdParams p) {
  constexpr int BM = NWV * RW;
  constexpr int RBW = RW / 16;       // 16-row blocks per wave
  constexpr int KB = BN / 16;        // 16-key blocks per tile
  constexpr int KS = DQK / 32;       // k-steps over d_qk
  constexpr int DB = DV / 16;        // 16-wide output column blocks
  constexpr int KRB = DQK * 2, VRB = DV * 2;   // bytes per K / V row
  constexpr bool PIPE = DQK <= 128 && DV <= 128;   // operand reads one step ahead
  static_assert(KB % 2 == 0, "PV consumes keys in pairs of 16-key blocks");
  static_assert(NST >= 2 && BN <= 64, "ring of at least two stages; gate copy is one lane per key");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[NST][BN * KRB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[NST][BN * VRB];
  __shared__ __attribute__((aligned(16))) float gk_lds[NST][NWV][64];   // one copy per wave

  const int h = xcd_head(blockIdx.x, p.Hq), n = blockIdx.z;
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
      gq[rb] = GATED ? p.G2[(long)h * p.T + seq0 + row] : 0.f;
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
  // LDS by direct copies, NST-1 tiles ahead of the math, into a ring of NST
  // stages.  A tile of BN rows is NI 1 KB blocks; wave w copies blocks w,
  // w+4, ...  Lane l of block j holds bytes 16 l .. 16 l + 15 of the block:
  // tile row (1024 j + 16 l) / RB, logical chunk (position ^ swizzle).  Its
  // global offset from the tile's first row is fixed, so it is computed
  // once; only the last tile of the sequence clamps rows past the end to
  // the last row (in range and finite; those keys are masked).  Every wave
  // issues the same number of copies per tile, so the wait for the oldest
  // tile is an exact vmcnt.
  constexpr int KPW = BN * KRB / (NWV * 1024), VPW = BN * VRB / (NWV * 1024);   // blocks per wave
  constexpr int LOADS_PER_TILE = KPW + VPW + (GATED ? 1 : 0);
  static_assert(KPW * NWV * 1024 == BN * KRB && VPW * NWV * 1024 == BN * VRB,
                "tile must split into NWV x k 1 KB blocks");
  int krow[KPW], koff[KPW], vrow[VPW], voff[VPW];
#pragma unroll
  for (int j = 0; j < KPW; ++j) {
    const int o = (wave + NWV * j) * 1024 + lane * 16;
    krow[j] = o / KRB;
    koff[j] = (int)(krow[j] * kstride) + ((((o % KRB) >> 4) ^ tile_swz<KRB>(krow[j])) << 4);
  }
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int o = (wave + NWV * j) * 1024 + lane * 16;
    vrow[j] = o / VRB;
    voff[j] = (int)(vrow[j] * vstride) + ((((o % VRB) >> 4) ^ tile_swz<VRB>(vrow[j])) << 4);
  }
  const float* g2base = GATED ? p.G2 + (long)h * p.T + seq0 : nullptr;
  auto fetch = [&](int st, int j0) {
    const bool tail = j0 + BN > L;         // uniform: only the last tile clamps
    const uint8_t* kb = kbase + j0 * kstride;
    const uint8_t* vb = vbase + j0 * vstride;
    const uint32_t kl = lds_addr(k_lds[st]), vl = lds_addr(v_lds[st]);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int over = tail ? max(0, j0 + krow[j] - (L - 1)) : 0;
      dma16(kb, (uint32_t)(koff[j] - over * (int)kstride), kl + (wave + NWV * j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int over = tail ? max(0, j0 + vrow[j] - (L - 1)) : 0;
      dma16(vb, (uint32_t)(voff[j] - over * (int)vstride), vl + (wave + NWV * j) * 1024);
    }
    if constexpr (GATED)
      dma4(g2base, (uint32_t)(min(j0 + lane, L - 1) * 4), lds_addr(&gk_lds[st][wave][0]));
  };

  // Per-lane LDS offsets of the operands this lane reads (a row's swizzle
  // depends only on its index mod 16): K rows kb*16 + li at k-step ks, V^T
  // rows kp*32 + 4g + mm (and 16 below) at output block db.
  const int mm = li >> 2, c4 = li & 3;
  uint32_t k_lane[KS], v_lane[DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_lane[ks] = (uint32_t)tile_off<KRB>(li, 64 * ks + 16 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db) v_lane[db] = (uint32_t)tile_off<VRB>(4 * g + mm, 32 * db + 8 * c4);

  // prologue: tiles t_begin .. t_begin+NST-2
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (t_begin + s < t_end) fetch(s, (t_begin + s) * BN);

  // Every wave takes part in every tile's wait, barrier and copies ...
  auto sync = [&](int t) {
    // wait for tile t: the tiles issued after it that may still be in flight
    const int later = min(NST - 2, t_end - 1 - t);
    if (later <= 0) wait_vm<0>();
    else if (later == 1) wait_vm<LOADS_PER_TILE>();
    else wait_vm<2 * LOADS_PER_TILE>();
    lds_barrier();   // tile t visible to all waves; stage of tile t-1 free
    if (t + NST - 1 < t_end) fetch((t - t_begin + NST - 1) % NST, (t + NST - 1) * BN);
  };
  // ... but computes only the tiles its rows can see: [tw_lo, tw_hi), keys
  // from the first row's window start to the last row.  The three loops
  // keep the tile body free of a branch (a branch around it costs the
  // kernel registers and occupancy).  Inside the range, a tile that
  // crosses the diagonal, the window edge or the end is masked per element.
  int tw_lo = t_begin, tw_hi = t_end;
  {
    if (W > 0 && r0 - W + 1 > 0) tw_lo = max(t_begin, (r0 - W + 1) / BN);
    tw_hi = r_last >= r0 ? min(t_end, r_last / BN + 1) : t_begin;
    tw_lo = min(tw_lo, tw_hi);
  }
  for (int t = t_begin; t < tw_lo; ++t) sync(t);
  for (int t = tw_lo; t < tw_hi; ++t) {
    const int j0 = t * BN;
    const int st = (t - t_begin) % NST;
    sync(t);
    {
      const bool need_mask = (j0 + BN - 1 > r0) || (W > 0 && r_last - j0 >= W) || (j0 + BN > L) ||
                             (r_last < r0 + RW - 1);
      // (the empty asm keeps each per-tile address whole, so that the
      // compiler folds the constant parts into the reads' offset fields
      // instead of hoisting one register per read out of the loop)
      const uint32_t kst = lds_addr(k_lds[st]), vst = lds_addr(v_lds[st]);
      const LDS_AS uint8_t* ka[KS];
      const LDS_AS uint8_t* va[DB];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t a = kst + k_lane[ks];
        asm volatile("" : "+v"(a));
        ka[ks] = (const LDS_AS uint8_t*)a;
      }
      const float* gkl = gk_lds[st][wave];
      // ---- S^T = K Q^T ----
      // Head dims up to 128 (PIPE): operand reads run one step ahead, the K
      // fragments of key block kb+1 read while block kb's MFMAs run, so the
      // LDS latency hides behind a block of MFMAs instead of stalling every
      // pair (the scheduling fences keep that order; measured ~2 % on the
      // 8-sequence window-1024 workload).  Wider heads keep the plain order:
      // the extra fragments would cost them occupancy.
      f32x4 sc[KB][RBW];
      constexpr int VG = DB < 4 ? DB : 4;           // output blocks per PV group
      constexpr int NGV = (KB / 2) * (DB / VG);     // PV groups per tile
      bf16x8 vf[2][VG];
      if constexpr (PIPE) {
        bf16x8 kf[2][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[0][ks] = *reinterpret_cast<const LDS_AS bf16x8*>(ka[ks]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (kb + 1 < KB) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              kf[(kb + 1) & 1][ks] = *reinterpret_cast<const LDS_AS bf16x8*>(ka[ks] + (kb + 1) * 16 * KRB);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = mfma16x16x32(kf[kb & 1][ks], qop[rb][ks], sc[kb][rb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // V^T addresses, and the first group of V^T fragments read now so
        // that their latency hides behind the softmax
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          uint32_t a = vst + v_lane[db];
          asm volatile("" : "+v"(a));
          va[db] = (const LDS_AS uint8_t*)a;
        }
#pragma unroll
        for (int j = 0; j < VG; ++j) vf[0][j] = concat(lds_tr16(va[j]), lds_tr16(va[j] + 16 * VRB));
        __builtin_amdgcn_sched_barrier(0);
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const LDS_AS bf16x8*>(ka[ks] + kb * 16 * KRB);
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) sc[kb][rb] = mfma16x16x32(a, qop[rb][ks], sc[kb][rb]);
          }
        }
      }
      // ---- gated: y = s*c - gk (base 2, without the row's gate term);
      //      ungated scores stay raw until the exponent (c > 0, so the
      //      max commutes with the scaling) ----
      if constexpr (GATED) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const f32x4 gk = *reinterpret_cast<const f32x4*>(gkl + kb * 16 + 4 * g);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[kb][rb][i] = __builtin_fmaf(sc[kb][rb][i], c, -gk[i]);
        }
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
        float mx = tile_row_max<KB>(sc, rb);
        mx = xgroup_max(mx);
        if constexpr (!GATED) mx *= c;
        if (__builtin_expect(__any(mx > m_run[rb] + kRescaleSlack), 0)) {
          const float m_new = fmaxf(m_run[rb], mx);
          const float alpha = fast_exp2(m_run[rb] - m_new);
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
          m_run[rb] = m_new;
        }
        const float mr = m_run[rb];
        float part[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          f32x4 e;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            e[i] = fast_exp2(GATED ? sc[kb][rb][i] - mr : __builtin_fmaf(sc[kb][rb][i], c, -mr));
          part[kb] = (e[0] + e[1]) + (e[2] + e[3]);
          pb[kb][rb] = to_bf16x4(e);
        }
        const float rs = tree_sum<KB>(part);
        l_run[rb] += xgroup_sum(rs);   // fp32 row sum: lse feeds the backward
      }
      // ---- O^T += V^T P^T, 32 keys per MFMA ----
      if constexpr (PIPE) {
        // in groups of VG output blocks; group n+1's fragments are read
        // while group n's MFMAs run
#pragma unroll
        for (int n = 0; n < NGV; ++n) {
          const int kp = n / (DB / VG), db0 = (n % (DB / VG)) * VG;
          if (n + 1 < NGV) {
            const int kp1 = (n + 1) / (DB / VG), db1 = ((n + 1) % (DB / VG)) * VG;
#pragma unroll
            for (int j = 0; j < VG; ++j)
              vf[(n + 1) & 1][j] = concat(lds_tr16(va[db1 + j] + kp1 * 32 * VRB),
                                          lds_tr16(va[db1 + j] + (kp1 * 32 + 16) * VRB));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < VG; ++j)
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
              oacc[rb][db0 + j] =
                  mfma16x16x32(vf[n & 1][j], concat(pb[2 * kp][rb], pb[2 * kp + 1][rb]), oacc[rb][db0 + j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          uint32_t a = vst + v_lane[db];
          asm volatile("" : "+v"(a));
          va[db] = (const LDS_AS uint8_t*)a;
        }
#pragma unroll
        for (int kp = 0; kp < KB / 2; ++kp) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = concat(lds_tr16(va[db] + kp * 32 * VRB), lds_tr16(va[db] + (kp * 32 + 16) * VRB));
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
              oacc[rb][db] = mfma16x16x32(a, concat(pb[2 * kp][rb], pb[2 * kp + 1][rb]), oacc[rb][db]);
          }
        }
      }
    }
  }
  for (int t = tw_hi; t < t_end; ++t) sync(t);

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

template <int DQK, int DV, int RW, int BN, int NST, int NWV = 4>
static hipError_t launch_cfg(const FwdParams& p, hipStream_t st) {
  constexpr int BM = NWV * RW;
  const int tiles = (p.max_seqlen + BM - 1) / BM;
  dim3 grid(p.Hq, tiles, p.num_seqs), block(64 * NWV);   // sequence-major: a sequence's tiles share L2
  if (p.G2 != nullptr)
    fwd_kernel<DQK, DV, RW, BN, NST, true, NWV><<<grid, block, 0, st>>>(p);
  else
    fwd_kernel<DQK, DV, RW, BN, NST, false, NWV><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace attn
