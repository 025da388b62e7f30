// Paged prefill as a pipelined tile loop: whole 64-key tiles of the paged
// cache in the bf16 tile that the forward's 32x32x16 MFMA body reads (an
// fp8 cache converted into it once per workgroup).
//
// Method (ROCm/aiter PR #6660, "Technical details" and commit messages 2
// and 3; fla issue #1322, Description, for the causal online softmax): the
// rows are the new tokens of a request, token t at position L - n + t,
// seeing the keys up to its own position (and inside the window); each
// score column is scaled by its key's K scale, and once the row sum has
// been taken each probability column is scaled by its key's V scale before
// the value product, that product carried as a bf16 high part plus a bf16
// low part (so the fp8 path keeps the precision of its fp32 P).  Per-tensor
// scales fold the K scale into the score factor and apply the V scale to
// the output; a bf16 cache has no scales and its P enters PV as one bf16.
// The sink logit joins the softmax denominator without a value; the log-gate
// bias G(query position) - G(key) comes from the paged cumulative-gate cache
// [pages, query heads, page size].
//
// gfx950 mapping (the tile body of fwd_pipe.h, adapted):
//  * One workgroup of four waves per (HPW query heads of one KV group,
//    query tile, request); wave w takes head w % HPW and 32 tokens.
//  * Per 64-key tile every wave copies its quarter of the K and V rows from
//    their pages (global_load_lds from the page base in SGPRs, one tile
//    ahead).  fp8: into a raw LDS ring, then the wave converts exactly the
//    bytes it copied into the swizzled bf16 tile (v_cvt_scalef32_pk_bf16_fp8:
//    exact, scale 1), and the workgroup synchronises twice per tile (before
//    the conversion, the bf16 tile being free, and after it).  bf16: straight
//    into a two-stage ring of swizzled tiles, one barrier per tile.  V rows
//    past the sequence end are zeroed (their cache bytes may be NaN).
//  * Sᵀ = K Qᵀ and Oᵀ += Vᵀ Pᵀ on v_mfma_f32_32x32x16_bf16 with the
//    exponentials of the previous tile between the QK MFMAs and the V-scaled
//    high / low parts of its probabilities formed between the PV MFMAs.
#include "fwd_pipe.h"

namespace attn {

namespace {

// 8 e4m3fn bytes -> 8 bf16 (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_bf16(i32x2 w) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Cache modes: fp8 with per-token scales, fp8 with per-tensor scales, bf16.
constexpr int kPagedFp8Token = 0, kPagedFp8Tensor = 1, kPagedBf16 = 2;

template <int D, int HPW, int MODE, bool GATED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void paged_pipe_kernel(DecodeParams p) {
  constexpr bool FP8 = MODE != kPagedBf16;
  constexpr bool PT = MODE == kPagedFp8Tensor;
  constexpr bool SCALES = MODE == kPagedFp8Token;   // per-key K / V scales, P' as high + low parts
  constexpr int RW = 32;                 // tokens per wave
  constexpr int WPH = 4 / HPW;           // row groups per head
  constexpr int BM = RW * WPH;           // tokens per workgroup
  constexpr int BN = 64, KB = BN / 32;   // keys per tile, 32-key blocks per tile
  constexpr int KS = D / 16;             // QK k-steps
  constexpr int DB = D / 32;             // 32-wide output column blocks
  constexpr int PS = BN / 16;            // PV k-steps
  constexpr int RB = D * 2;              // bytes per bf16 tile row
  constexpr int CROW = FP8 ? D : 2 * D;  // bytes per cache row
  constexpr int KPC = 1024 / CROW;       // keys per 1 KB copy
  constexpr int NCP = BN / KPC;          // copies per tile and tensor
  constexpr int CPW = NCP / 4;           // ... per wave
  constexpr int LPR = CROW / 16;         // lanes per cache row in a copy
  static_assert(CPW * 4 == NCP && CPW >= 1, "tile copies split over four waves");
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  constexpr int NQK = KB * KS, NPV = PS * DB, NE = KB * 16;
  constexpr int NSTB = FP8 ? 1 : 2;      // bf16 tile stages
  constexpr int RAW = FP8 ? BN * CROW : 16;
  constexpr int NSC = SCALES ? BN : 4;
  constexpr int NGK = GATED ? BN : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[NSTB][BN * RB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[NSTB][BN * RB];
  __shared__ __attribute__((aligned(1024))) uint8_t kr_lds[2][RAW];   // fp8: raw tiles
  __shared__ __attribute__((aligned(1024))) uint8_t vr_lds[2][RAW];
  __shared__ __attribute__((aligned(16))) float ks_lds[2][NSC];       // K scale * score factor per key
  __shared__ __attribute__((aligned(16))) float vs_lds[2][NSC];       // V scale per key
  __shared__ __attribute__((aligned(16))) float gk_lds[2][4][NGK];    // per wave: -log2(e) G of its head's keys

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, hh = lane >> 5;
  const int G = p.Hq / p.Hkv;
  const int hx = xcd_group(blockIdx.x, p.Hq / HPW);
  const int h = hx * HPW + wave % HPW;
  const int kvh = __builtin_amdgcn_readfirstlane((hx * HPW) / G);   // the workgroup's heads share it
  const int r = blockIdx.z;
  const int qs = p.cu_q[r];
  const int n = p.cu_q[r + 1] - qs;
  const int L = p.seq_lens[r];
  const int i0 = blockIdx.y * BM;
  if (i0 >= n) return;
  const int P0 = L - n;                  // position of the request's first new token
  const int W = p.window;
  const int bsh = p.B_shift, bmask = p.B - 1;
  const int32_t* bt = p.block_table + (long)r * p.max_pages;
  // score factor (log2 units); per-tensor K scale folded in
  const float c = PT ? p.scale_log2 * p.k_scale[0] : p.scale_log2;
  const float v_mul = PT ? p.v_scale[0] : 1.f;

  const int t0 = i0 + (wave / HPW) * RW;       // first token of this wave
  const int t_last = min(t0 + RW, n) - 1;      // last real token (may be < t0)
  const int tok = t0 + lr;                     // this lane's token
  const int pos = P0 + tok;                    // its position
  const int pos0 = P0 + t0, pos_last = P0 + t_last;

  // ---- Q operand and per-row state ----
  bf16x8 qop[KS];
  if (tok < n) {
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + ((long)(qs + tok) * p.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = bf16x8{};
  }
  // gate of the row's own position (the query side of G_query - G_key);
  // the running max is kept without it
  float gq = 0.f;
  if constexpr (GATED) {
    const int pr = min(pos, L - 1);
    const int pq = bt[pr >> bsh];
    gq = p.g_cache[((((long)pq * p.Hq + h) << bsh) + (pr & bmask))] * kLog2e;
  }
  float m_run = p.sink ? p.sink[h] * kLog2e - gq : kNegBig;
  float l_run = p.sink ? 1.f : 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // ---- key range of the workgroup and of this wave ----
  const int kv_lo = W > 0 ? max(0, P0 + i0 - W + 1) : 0;
  const int kv_hi = min(L, P0 + min(i0 + BM, n));   // one past the last visible key
  const int t_begin = kv_lo / BN, t_end = (kv_hi + BN - 1) / BN;
  int tw_lo = t_begin, tw_hi = t_begin;
  if (t_last >= t0) {
    tw_lo = (W > 0 && pos0 - W + 1 > 0) ? max(t_begin, (pos0 - W + 1) / BN) : t_begin;
    tw_hi = min(t_end, pos_last / BN + 1);
    tw_lo = min(tw_lo, tw_hi);
  }

  // ---- copies.  Copy cb of a tile holds KPC consecutive keys (one page
  // holds them: pages are whole multiples of KPC keys); wave w issues copies
  // w, w + 4, ...  Groups past the last key re-read the group of the last
  // key (in range; those rows are zeroed at conversion). ----
  const int last_group = ((L - 1) / KPC) * KPC;
  const uint8_t* kcache = reinterpret_cast<const uint8_t*>(p.k_cache);
  const uint8_t* vcache = reinterpret_cast<const uint8_t*>(p.v_cache);
  auto group_base = [&](const uint8_t* cache, int k0) {
    const int kc = __builtin_amdgcn_readfirstlane(min(k0, last_group));
    const int page = bt[kc >> bsh];   // wave-uniform: a scalar load
    return sgpr_ptr(cache + (((long)page * p.Hkv + kvh) * p.B + (kc & bmask)) * CROW);
  };
  // one value per key of the tile, lane l -> key min(j0 + l, L - 1), from
  // the (at most four) pages the tile spans: the element offset of slot
  // (page, head hd of nh, key) in a [pages, nh, page size] array
  auto slot_off = [&](int j0, int nh, int hd) {
    const int key = min(j0 + lane, L - 1);
    const int pi0 = j0 >> bsh;
    const int last_pi = (L - 1) >> bsh;
    const int q = (key >> bsh) - pi0;   // 0 .. 3
    const int pa = bt[min(pi0, last_pi)], pb = bt[min(pi0 + 1, last_pi)];
    const int pc = bt[min(pi0 + 2, last_pi)], pd = bt[min(pi0 + 3, last_pi)];
    const int page = q == 0 ? pa : q == 1 ? pb : q == 2 ? pc : pd;
    return ((((uint32_t)page * (uint32_t)nh + (uint32_t)hd) << bsh) + (uint32_t)(key & bmask)) * 4u;
  };
  // bf16 copies land in the swizzled tile directly: lane l fills bytes
  // 16 l .. 16 l + 15 of its 1 KB block, tile row KPC cb + l / (RB / 16) at
  // chunk position l % (RB / 16), which holds logical chunk position ^ swz
  auto src_off = [&](int cb, bool is_v) -> uint32_t {
    if constexpr (FP8) return (uint32_t)(lane * 16);
    const int rr = lane / (RB / 16), pc = lane % (RB / 16);
    const int row = KPC * cb + rr;
    const int sw = is_v ? swz_v32<RB>(row) : swz_k32<RB>(row);
    return (uint32_t)(rr * CROW + ((pc ^ sw) << 4));
  };
  // K of tile t (with its K scales and this wave's gate terms) -> stage t & 1
  auto fetch_k = [&](int t) {
    const int j0 = t * BN, st = t & 1;
    uint8_t* dst = FP8 ? kr_lds[st] : k_lds[st & (NSTB - 1)];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int cb = wave + 4 * j;
      dma16(group_base(kcache, j0 + KPC * cb), src_off(cb, false), lds_addr(dst + cb * 1024));
    }
    if constexpr (SCALES) {
      if (wave == 0) dma4(p.k_scale, slot_off(j0, p.Hkv, kvh), lds_addr(&ks_lds[st][0]));
    }
    if constexpr (GATED) dma4(p.g_cache, slot_off(j0, p.Hq, h), lds_addr(&gk_lds[st][wave][0]));
  };
  // V of tile t (with its V scales) -> stage t & 1
  auto fetch_v = [&](int t) {
    const int j0 = t * BN, st = t & 1;
    uint8_t* dst = FP8 ? vr_lds[st] : v_lds[st & (NSTB - 1)];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int cb = wave + 4 * j;
      dma16(group_base(vcache, j0 + KPC * cb), src_off(cb, true), lds_addr(dst + cb * 1024));
    }
    if constexpr (SCALES) {
      if (wave == 1) dma4(p.v_scale, slot_off(j0, p.Hkv, kvh), lds_addr(&vs_lds[st][0]));
    }
  };

  // ---- conversion of the bytes this wave copied: lane l of copy cb holds
  // 16 bytes of key KPC cb + l / LPR at dims 16 (l % LPR) .. + 15, i.e. the
  // bf16 chunks 2 (l % LPR) and 2 (l % LPR) + 1 of that tile row ----
  auto convert = [&](const uint8_t* raw, uint8_t* tile, int j0, bool is_v) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int cb = wave + 4 * j;
      const int row = KPC * cb + lane / LPR;
      const int lc = 2 * (lane % LPR);
      const i32x4 w = *reinterpret_cast<const i32x4*>(raw + cb * 1024 + lane * 16);
      bf16x8 lo8 = fp8x8_bf16(i32x2{w[0], w[1]});
      bf16x8 hi8 = fp8x8_bf16(i32x2{w[2], w[3]});
      if (j0 + row >= L) {   // past the sequence end: the cache bytes may be NaN
        lo8 = bf16x8{};
        hi8 = bf16x8{};
      }
      const int sw = is_v ? swz_v32<RB>(row) : swz_k32<RB>(row);
      *reinterpret_cast<bf16x8*>(tile + row * RB + (((lc) ^ sw) << 4)) = lo8;
      *reinterpret_cast<bf16x8*>(tile + row * RB + (((lc + 1) ^ sw) << 4)) = hi8;
    }
  };
  // K scales of tile t times the score factor, in place (wave 0 reads back
  // the element its own lane copied); clamped away from 0 so that a masked
  // score (-inf) stays -inf
  auto scale_k = [&](int t) {
    if constexpr (SCALES) {
      if (wave == 0) {
        float* s = &ks_lds[t & 1][lane];
        *s = fmaxf(*s * c, 1e-30f);
      }
    }
    if constexpr (GATED) {   // the wave's own gate terms, times -log2(e)
      float* g = &gk_lds[t & 1][wave][lane];
      *g = *g * -kLog2e;
    }
  };
  // bf16: V rows past the sequence end that this wave copied (stage of tile t)
  auto zero_tail_v = [&](int t) {
    if constexpr (!FP8) {
      const int j0 = t * BN;
      if (j0 + BN > L) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const int cb = wave + 4 * j;
          const int row = KPC * cb + lane / (RB / 16);
          if (j0 + row >= L) *reinterpret_cast<i32x4*>(v_lds[t & (NSTB - 1)] + cb * 1024 + lane * 16) = i32x4{0, 0, 0, 0};
        }
      }
    }
  };

  // ---- per-lane LDS operand addresses (as in fwd_pipe.h) ----
  const uint32_t k_lane0 = (uint32_t)(lr * RB + ((hh ^ swz_k32<RB>(lr)) << 4));
  const int vj = (lane & 15) >> 2, vc = lane & 3, vhalf = (lane >> 4) & 1;
  const int vrow = 4 * hh + vj;
  const uint32_t v_lane0 =
      (uint32_t)(vrow * RB + (((2 * vhalf + (vc >> 1)) ^ swz_v32<RB>(vrow)) << 4) + 8 * (vc & 1));
  auto k_addr = [&](int t, int ks) {
    uint32_t a = (lds_addr(k_lds[t & (NSTB - 1)]) + k_lane0) ^ (uint32_t)(32 * ks);
    asm volatile("" : "+v"(a));
    return (const LDS_AS uint8_t*)a;
  };
  auto v_addr = [&](int t, int db) {
    uint32_t a = (lds_addr(v_lds[t & (NSTB - 1)]) + v_lane0) ^ (uint32_t)(64 * db);
    asm volatile("" : "+v"(a));
    return (const LDS_AS uint8_t*)a;
  };

  // ---- iteration t: K(t) and V(t-1) become bf16 tiles; K(t+1), V(t) go
  // in flight.  Every wave takes part in every iteration t_begin .. t_end.
  fetch_k(t_begin);
  auto sync = [&](int t) {
    wait_vm<0>();
    if constexpr (FP8) {
      lds_barrier();   // everyone past iteration t-1: the bf16 tiles are free
      if (t < t_end) {
        convert(kr_lds[t & 1], k_lds[0], t * BN, false);
        scale_k(t);
      }
      if (t > t_begin) convert(vr_lds[(t - 1) & 1], v_lds[0], (t - 1) * BN, true);
      if (t + 1 < t_end) fetch_k(t + 1);
      if (t < t_end) fetch_v(t);
      lds_barrier();   // converted tiles and scales visible
    } else {
      if (t < t_end) scale_k(t);
      if (t > t_begin) zero_tail_v(t - 1);
      lds_barrier();   // tiles K(t), V(t-1) landed everywhere; the stages of K(t-1), V(t-2) are free
      if (t + 1 < t_end) fetch_k(t + 1);
      if (t < t_end) fetch_v(t);
    }
  };

  auto mask = [&](int t, f32x16 (&s)[KB]) {
    asm volatile("" ::: "memory");
    const int j0 = t * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = j0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool vis = key <= pos && key < L && (W <= 0 || pos - key < W);
        s[kb][i] = vis ? s[kb][i] : -INFINITY;
      }
  };
  auto need_mask = [&](int t) {
    const int j0 = t * BN;
    return (j0 + BN - 1 > pos0) || (W > 0 && pos_last - j0 >= W) || (j0 + BN > L) || (t_last < t0 + RW - 1);
  };
  float mx = -INFINITY;
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

  // Exponent work (block A) on y (the previous tile), in place; every 8
  // elements add their sum to the row sum.  The row sum is of P itself.
  float rsum = 0.f;
  auto exp_elem = [&](f32x16 (&y)[KB], int e) { y[e / 16][e % 16] = fast_exp2(y[e / 16][e % 16] - m_run); };
  auto exp_group = [&](f32x16 (&y)[KB], int gi) {
    const int kb = gi / 2, o = 8 * (gi % 2);
    const float pt = ((y[kb][o] + y[kb][o + 1]) + (y[kb][o + 2] + y[kb][o + 3])) +
                     ((y[kb][o + 4] + y[kb][o + 5]) + (y[kb][o + 6] + y[kb][o + 7]));
    rsum = gi == 0 ? pt : rsum + pt;
  };
  auto exp_row = [&]() {
    const unsigned u = __float_as_uint(rsum);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    l_run += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
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

  // P operand of PV k-step ps (keys 16 ps + 8 (e / 4) + 4 hh + e % 4): the
  // probabilities times their V scales as bf16 high and low parts (one
  // rounding each: hi = RNE(P'), lo = RNE(P' - hi)); per-tensor scales: P.
  bf16x8 phi[2], plo[2];
  const SplitCoef coef = split_coef();
  auto p_operand = [&](f32x16 (&y)[KB], int ps, int t_v) {
    const int kb = ps / 2, o = 8 * (ps % 2);
    float a[8];
    if constexpr (!SCALES) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = y[kb][o + e];
    } else {
      const float* vs = &vs_lds[t_v & 1][32 * kb + 4 * hh];
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(vs + 8 * (o / 4));
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(vs + 8 * (o / 4 + 1));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = y[kb][o + e] * v0[e];
        a[e + 4] = y[kb][o + 4 + e] * v1[e];
      }
    }
    bf16x8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 hp = __builtin_convertvector(f32x2{a[e], a[e + 1]}, bf16x2);
      hv[e] = hp[0];
      hv[e + 1] = hp[1];
      if constexpr (SCALES) {
        const bf16x2 lp = __builtin_convertvector(split_lo(hp, a[e], a[e + 1], coef), bf16x2);
        lv[e] = lp[0];
        lv[e + 1] = lp[1];
      }
    }
    phi[ps & 1] = hv;
    if constexpr (SCALES) plo[ps & 1] = lv;
  };

  // Bias work (block B) on the fresh scores s: s * (K scale * factor), in
  // place, and the running row max.
  f32x4 ks4[2];
  const float* ksl = nullptr;
  float mrow = -INFINITY;
  auto ks_read = [&](int gi) {
    if constexpr (SCALES) ks4[gi & 1] = *reinterpret_cast<const f32x4*>(ksl + 8 * gi + 4 * hh);
  };
  f32x4 gk4[2];
  const float* gkl = nullptr;
  auto gk_read = [&](int gi) {
    if constexpr (GATED) gk4[gi & 1] = *reinterpret_cast<const f32x4*>(gkl + 8 * gi + 4 * hh);
  };
  auto bias_elem = [&](f32x16 (&s)[KB], int e) {
    const int kb = e / 16, i = e % 16, gi = e / 4;
    if (i % 4 == 0 && gi + 1 < NE / 4) {
      ks_read(gi + 1);
      gk_read(gi + 1);
    }
    const float f = SCALES ? ks4[gi & 1][i % 4] : c;
    if constexpr (GATED) s[kb][i] = __builtin_fmaf(s[kb][i], f, gk4[gi & 1][i % 4]);
    else s[kb][i] = s[kb][i] * f;
  };
  auto bias_slot = [&](f32x16 (&s)[KB], int j, auto ns) {
    constexpr int per = NE / decltype(ns)::value;
#pragma unroll
    for (int q = 0; q < per; ++q) bias_elem(s, j * per + q);
    if (j > 0) {
      const int e0 = (j - 1) * per;
#pragma unroll
      for (int e = 0; e < per; ++e) mrow = fmaxf(mrow, s[(e0 + e) / 16][(e0 + e) % 16]);
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
    if constexpr (SCALES) {
      ksl = &ks_lds[t & 1][0];
      ks_read(0);
    }
    if constexpr (GATED) {
      gkl = &gk_lds[t & 1][wave][0];
      gk_read(0);
    }
    mrow = -INFINITY;
  };

  // Block A: S(t) = K(t) Q^T, with the exponent work of yold between the MFMAs.
  constexpr int FA_LEAD = SCALES ? 2 : 3, FA_NB = FA_LEAD + 1;   // per-token scales hold two P' operands
  auto block_a = [&](int t, f32x16 (&snew)[KB], f32x16 (&yold)[KB], bool ex) {
    const LDS_AS uint8_t* ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = k_addr(t, ks);
    bf16x8 kf[FA_NB];
    auto kread = [&](int f) { kf[f % FA_NB] = *reinterpret_cast<const LDS_AS bf16x8*>(ka[f % KS] + (f / KS) * 32 * RB); };
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
  // Block B: O^T += V^T(t-1) P'^T (high and low parts) slot by slot, with the
  // next k-step's P' operand and the bias and max work of s between the
  // MFMAs; V^T fragments are read FB_LEAD slots ahead.
  constexpr int FB_LEAD = SCALES ? 1 : 2, FB_NB = FB_LEAD + 1;
  auto pv_mfma = [&](const bf16x8& a, int ps, int db) {
    oacc[db] = mfma32x32x16(a, phi[ps & 1], oacc[db]);
    if constexpr (SCALES) oacc[db] = mfma32x32x16(a, plo[ps & 1], oacc[db]);
  };
  auto block_b = [&](int t, f32x16 (&s)[KB], f32x16 (&yold)[KB], bool pvon) {
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
    auto vread = [&](int f) {
      const int ps = f / DB, db = f % DB;
      vf[f % FB_NB] = concat(lds_tr16(va[db] + 16 * ps * RB), lds_tr16(va[db] + (16 * ps + 8) * RB));
    };
#pragma unroll
    for (int f = 0; f < FB_LEAD && f < NPV; ++f) vread(f);
    p_operand(yold, 0, t - 1);
#pragma unroll
    for (int sl = 0; sl < NPV; ++sl) {
      const int ps = sl / DB, db = sl % DB;
      if (sl + FB_LEAD < NPV) vread(sl + FB_LEAD);
      pv_mfma(vf[sl % FB_NB], ps, db);
      if (db == 0 && ps + 1 < PS) p_operand(yold, ps + 1, t - 1);
      bias_slot(s, sl, std::integral_constant<int, NPV>{});
      __builtin_amdgcn_sched_barrier(0);
    }
    bias_tail(s, std::integral_constant<int, NPV>{});
  };
  // plain PV (epilogue) of tile t - 1
  auto pv_only = [&](int t, f32x16 (&yold)[KB]) {
    const LDS_AS uint8_t* va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = v_addr(t - 1, db);
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      p_operand(yold, ps, t - 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a = concat(lds_tr16(va[db] + 16 * ps * RB), lds_tr16(va[db] + (16 * ps + 8) * RB));
        pv_mfma(a, ps, db);
      }
    }
  };

  f32x16 sA[KB], sB[KB];
  auto first = [&](int t, f32x16 (&s)[KB]) {
    sync(t);
    block_a(t, s, sB, false);
    if (need_mask(t)) mask(t, s);
    block_b(t, s, sB, false);
    rescale();
  };
  auto full = [&](int t, f32x16 (&snew)[KB], f32x16 (&yold)[KB]) {
    sync(t);
    block_a(t, snew, yold, true);
    if (need_mask(t)) mask(t, snew);
    block_b(t, snew, yold, true);
    rescale();
  };
  auto last = [&](int t, f32x16 (&yold)[KB]) {
    sync(t);
#pragma unroll
    for (int j = 0; j < 16; ++j) exp_slot(yold, j, std::integral_constant<int, 16>{});
    exp_tail(yold, std::integral_constant<int, 16>{});
    pv_only(t, yold);
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

  // ---- output: O = v_mul acc / l, lse = ln 2 (m + log2 l) ----
  if (tok < n) {
    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : v_mul / l_run;
    const long grow = (long)(qs + tok) * p.Hq + h;
    bf16* op = reinterpret_cast<bf16*>(p.out) + grow * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = f32x4{oacc[db][4 * q], oacc[db][4 * q + 1], oacc[db][4 * q + 2], oacc[db][4 * q + 3]} * inv;
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * q) = to_bf16x4(x);
      }
    if (hh == 0 && p.lse != nullptr) p.lse[grow] = empty ? -INFINITY : (m_run + gq + fast_log2(l_run)) * kLn2;
  }
}

template <int D, int HPW, int MODE>
hipError_t launch_paged_mode(const DecodeParams& p, int max_q, hipStream_t st) {
  constexpr int BM = 32 * (4 / HPW);
  const dim3 grid(p.Hq / HPW, (max_q + BM - 1) / BM, p.R);
  if (p.g_cache != nullptr)
    paged_pipe_kernel<D, HPW, MODE, true><<<grid, 256, 0, st>>>(p);
  else
    paged_pipe_kernel<D, HPW, MODE, false><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, int HPW>
hipError_t launch_paged_hpw(const DecodeParams& p, bool fp8, int max_q, hipStream_t st) {
  if (!fp8) return launch_paged_mode<D, HPW, kPagedBf16>(p, max_q, st);
  if (p.per_tensor) return launch_paged_mode<D, HPW, kPagedFp8Tensor>(p, max_q, st);
  return launch_paged_mode<D, HPW, kPagedFp8Token>(p, max_q, st);
}

template <int D>
hipError_t launch_paged_d(const DecodeParams& p, bool fp8, int max_q, hipStream_t st) {
  const int grp = p.Hq / p.Hkv;
  if (grp % 4 == 0) return launch_paged_hpw<D, 4>(p, fp8, max_q, st);
  if (grp % 2 == 0) return launch_paged_hpw<D, 2>(p, fp8, max_q, st);
  return launch_paged_hpw<D, 1>(p, fp8, max_q, st);
}

}  // namespace

bool paged_pipe_supported(const DecodeParams& p, int head_dim, bool fp8, float softmax_scale) {
  // one copy holds 1024 bytes of consecutive keys of one page
  const int keys_per_copy = 1024 / (head_dim * (fp8 ? 1 : 2));
  return (head_dim == 64 || head_dim == 128) && p.num_splits == 1 && softmax_scale > 0.f &&
         p.B >= keys_per_copy && p.out != nullptr;
}

hipError_t launch_paged_pipe(const DecodeParams& p, int head_dim, bool fp8, int max_q, hipStream_t st) {
  if (head_dim == 128) return launch_paged_d<128>(p, fp8, max_q, st);
  if (head_dim == 64) return launch_paged_d<64>(p, fp8, max_q, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
