// Paged split-K decode partials for 1..4 query tokens per request over a
// bf16 or per-token-scaled fp8 e4m3fn KV cache.
//
// Method (ROCm/aiter PR #6660, commit messages and "Technical details"):
// the keys of a request are split into segments; each (request, KV head,
// segment) produces (acc, m, l) partials for all query rows of the request
// that share the KV head.  K scales multiply the QK columns; V scales
// multiply the probability columns after the row sum; the scaled
// probabilities are split into a bf16 high and low part so that PV keeps
// fp32 accuracy; cache slots past seq_len never contribute (their bytes and
// scales may be NaN, so they are selected away, not multiplied by 0).  A
// query whose last visible key precedes the segment stores an empty partial
// (m = -inf, l = 0).
//
// gfx950 mapping: one wavefront per work item, so four independent streams
// per workgroup and no barriers.  The wave walks its segment 32 keys at a
// time:
//   S^T (32 keys x 16 rows per row block) = K Q^T with
//     v_mfma_f32_16x16x32_bf16; K is fetched straight from the pages into
//     the A-operand layout (fp8 -> bf16 conversion is exact), Q stays in
//     registers as the B operand for the whole segment;
//   online softmax per query row in the base-2 domain;
//   O^T += V^T (P v_scale)^T, twice (bf16 high and low parts); V is staged
//     through LDS in page order and read back transposed with
//     ds_read_b64_tr_b8 (fp8) / ds_read_b64_tr_b16 (bf16).
// Query rows are (query token, head of the KV group) pairs, so GQA 16 with
// one token fills one 16-row block and 4 tokens fill four.
#include "common.h"
#include "kernels.h"

namespace attn {

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 w) {
  f32x2 a = fp8x2_to_f32<false>(w[0]), b = fp8x2_to_f32<true>(w[0]);
  f32x2 c = fp8x2_to_f32<false>(w[1]), d = fp8x2_to_f32<true>(w[1]);
  return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)b[0], (bf16)b[1],
                (bf16)c[0], (bf16)c[1], (bf16)d[0], (bf16)d[1]};
}

__device__ __forceinline__ void lds_wave_sync() {
  // LDS operations of one wavefront complete in order; this only stops the
  // compiler from moving LDS accesses across the point and waits for them.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Raw bytes of one 32-key step, fetched one step ahead of their use.
template <int D, bool FP8>
struct StepRaw {
  static constexpr int ES = FP8 ? 1 : 2;
  static constexpr int KCH = (D / 4) * ES / 16;      // 16-byte K chunks per lane per key block
  static constexpr int NCH = 32 * D * ES / 16 / 64;  // 16-byte V chunks per lane
  i32x4 k[2][KCH];
  i32x4 v[NCH];
  f32x4 ks[2], vs[2];
};

template <int D, bool FP8, int RB>
__global__ __launch_bounds__(256) void decode_splitk_kernel(DecodeParams p) {
  using Raw = StepRaw<D, FP8>;
  constexpr int KS = D / 32;          // k-steps of 32 over the head dim
  constexpr int DPG = 8 * KS;         // head-dim elements per 16-lane group
  constexpr int ES = Raw::ES;         // bytes per cache element
  constexpr int ROWB = D * ES;        // bytes per cached token row
  constexpr int VROW = ROWB + 16;     // padded LDS row stride
  constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  constexpr int DB = D / 16;          // 16-wide output column blocks
  __shared__ __attribute__((aligned(16))) uint8_t v_lds_all[4][32 * VROW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  uint8_t* v_lds = v_lds_all[wave];

  long item = (long)blockIdx.x * 4 + wave;
  const int kvh = (int)(item % p.Hkv);
  item /= p.Hkv;
  const int r = (int)(item % p.R);
  const int s = (int)(item / p.R);
  if (s >= p.num_splits) return;
  const int L = p.seq_lens[r];
  const int k_begin = s * p.split_len;
  if (k_begin >= L) return;            // segment beyond this request: none
  const int k_end = min(L, k_begin + p.split_len);
  const int qs = p.cu_q[r];
  const int qlen = p.cu_q[r + 1] - qs;
  const int G = p.Hq / p.Hkv;
  const long head_stride = (long)p.B * D;              // elements per (page, kv head)
  const long page_stride = (long)p.Hkv * head_stride;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.k_cache) + kvh * head_stride * ES;
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.v_cache) + kvh * head_stride * ES;

  // Page ids are wave-uniform per 32-key step (a step spans at most two
  // pages, and one when pages hold 32 or more keys), so they come through
  // scalar loads, one step ahead of the vector loads that use them.  Keys
  // past seq_len read the request's last page and are masked later: every
  // load stays unconditional and in range, so several steps can be in flight.
  const int bsh = p.B_shift, bmask = p.B - 1;   // page size is a power of two
  const int last_page = (L - 1) >> bsh;
  const int32_t* bt = p.block_table + (long)r * p.max_pages;
  struct Pages { int a, b; };                    // pages of keys kk and kk+16
  auto pages_of = [&](int kk) {
    Pages pp;
    pp.a = __builtin_amdgcn_readfirstlane(bt[min(kk >> bsh, last_page)]);
    pp.b = __builtin_amdgcn_readfirstlane(bt[min((kk + 16) >> bsh, last_page)]);
    return pp;
  };

  auto fetch = [&](int kk, Pages pp, Raw& raw) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kk + kb * 16 + li;
      const long pid = kb ? pp.b : pp.a;
      const long off = (pid * page_stride + (long)(key & bmask) * D + g * DPG) * ES;
#pragma unroll
      for (int c = 0; c < Raw::KCH; ++c) raw.k[kb][c] = *reinterpret_cast<const i32x4*>(kc + off + 16 * c);
      if constexpr (FP8) {
        const int k4 = kk + kb * 16 + 4 * g;
        const long so = ((pid * p.Hkv + kvh) << bsh) + (k4 & bmask);
        raw.ks[kb] = *reinterpret_cast<const f32x4*>(p.k_scale + so);
        raw.vs[kb] = *reinterpret_cast<const f32x4*>(p.v_scale + so);
      }
    }
#pragma unroll
    for (int c = 0; c < Raw::NCH; ++c) {
      const int ch = lane + 64 * c;
      const int kr = ch / CPR, col = (ch % CPR) * 16;
      const int key = kk + kr;
      const long pid = kr < 16 ? pp.a : pp.b;
      const long off = (pid * page_stride + (long)(key & bmask) * D) * ES + col;
      raw.v[c] = *reinterpret_cast<const i32x4*>(vc + off);
    }
  };

  // Q rows as the B operand: lane (row li, group g) holds the head-dim
  // elements [g*DPG, g*DPG + DPG) in k-step order.
  bf16x8 qop[RB][KS];
  int pos[RB];
  bool rvalid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rho = rb * 16 + li;
    const int t = rho / G;
    rvalid[rb] = t < qlen;
    pos[rb] = L - qlen + t;
    if (rvalid[rb]) {
      const bf16* qp = reinterpret_cast<const bf16*>(p.q) +
                       ((long)(qs + t) * p.Hq + (long)kvh * G + rho % G) * D + g * DPG;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = *reinterpret_cast<const bf16x8*>(qp + 8 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = bf16x8{};
    }
  }

  f32x4 oacc[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegBig;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int kk, const Raw& raw) {
    // ---- V of the 32 keys into LDS, zeros past seq_len (NaN-safe select) ----
#pragma unroll
    for (int c = 0; c < Raw::NCH; ++c) {
      const int ch = lane + 64 * c;
      const int kr = ch / CPR, col = (ch % CPR) * 16;
      const i32x4 z = {0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(v_lds + kr * VROW + col) = (kk + kr < L) ? raw.v[c] : z;
    }
    // ---- scores S^T = K Q^T ----
    f32x4 sc[2][RB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kop[KS];
      if constexpr (FP8) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const i32x4 w = raw.k[kb][ks / 2];
          kop[ks] = fp8x8_to_bf16x8((ks & 1) ? i32x2{w[2], w[3]} : i32x2{w[0], w[1]});
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kop[ks] = __builtin_bit_cast(bf16x8, raw.k[kb][ks]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a = mfma16x16x32(kop[ks], qop[rb][ks], a);
        sc[kb][rb] = a;
      }
    }
    // ---- K scales on the score columns; mask (select: slots past seq_len may be NaN) ----
    float ksc[2][4], vsc[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = kk + kb * 16 + 4 * g + i < L;
        ksc[kb][i] = FP8 ? (ok ? raw.ks[kb][i] : 0.f) * p.scale_log2 : p.scale_log2;
        vsc[kb][i] = FP8 ? (ok ? raw.vs[kb][i] : 0.f) : 1.f;
      }
    // ---- online softmax; P' = P * v_scale split into bf16 hi + lo ----
    bf16x8 phi[RB], plo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float x[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kk + kb * 16 + 4 * g + i;
          const bool vis = key < L && key <= pos[rb];
          x[kb][i] = vis ? sc[kb][rb][i] * ksc[kb][i] : -INFINITY;
          mx = fmaxf(mx, x[kb][i]);
        }
      mx = xgroup_max(mx);
      if (__any(mx > m_run[rb] + kRescaleSlack)) {
        // raise the running max only when a score passes it by more than
        // the slack, so exp2(score - max) stays below 2^8 in between
        const float m_new = fmaxf(m_run[rb], mx);
        const float alpha = fast_exp2(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
        m_run[rb] = m_new;
      }
      const float m_new = m_run[rb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(x[kb][i] - m_new);
          rs += pv;
          const float pp = pv * vsc[kb][i];
          const bf16 h = (bf16)pp;
          phi[rb][kb * 4 + i] = h;
          plo[rb][kb * 4 + i] = (bf16)(pp - (float)h);
        }
      l_run[rb] += xgroup_sum(rs);
    }
    lds_wave_sync();
    // ---- O^T += V^T P'^T (hi and lo) ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 vop;
      if constexpr (FP8) {
        const int j = li >> 1, c = li & 1;
        const int row = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
        vop = fp8x8_to_bf16x8(lds_read_tr8(v_lds + row * VROW + db * 16 + 8 * c));
      } else {
        const int mm = li >> 2, c = li & 3;
        const bf16* b0 = reinterpret_cast<const bf16*>(v_lds + (4 * g + mm) * VROW) + db * 16 + 4 * c;
        const bf16* b1 = reinterpret_cast<const bf16*>(v_lds + (16 + 4 * g + mm) * VROW) + db * 16 + 4 * c;
        vop = concat(lds_read_tr16(b0), lds_read_tr16(b1));
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        oacc[rb][db] = mfma16x16x32(vop, phi[rb], oacc[rb][db]);
        oacc[rb][db] = mfma16x16x32(vop, plo[rb], oacc[rb][db]);
      }
    }
    lds_wave_sync();
  };

  if constexpr (RB <= 2) {
    // ---- two-deep software pipeline over 32-key steps ----
    // The prefetch is unconditional (its addresses are clamped in range):
    // a conditional one would make the compiler drain every outstanding
    // load at the branch join, serialising the pipeline.
    Raw ra, rb_;
    fetch(k_begin, pages_of(k_begin), ra);
    Pages nxt = pages_of(k_begin + 32);
    for (int kk = k_begin; kk < k_end; kk += 64) {
      fetch(kk + 32, nxt, rb_);
      nxt = pages_of(kk + 64);
      compute(kk, ra);
      if (kk + 32 >= k_end) break;
      fetch(kk + 64, nxt, ra);
      nxt = pages_of(kk + 96);
      compute(kk + 32, rb_);
    }
  } else {
    // Many query rows: more math per byte and no registers left for a
    // second buffer; fetch and compute one step at a time.
    Raw ra;
    for (int kk = k_begin; kk < k_end; kk += 32) {
      fetch(kk, pages_of(kk), ra);
      compute(kk, ra);
    }
  }

  // ---- store the partial ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rvalid[rb]) continue;
    const int rho = rb * 16 + li;
    const long grow = (long)(qs + rho / G) * p.Hq + (long)kvh * G + rho % G;
    float* a = p.acc + (grow * p.num_splits + s) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(a + db * 16 + 4 * g) = oacc[rb][db];
    if (g == 0) {
      const bool empty = !(l_run[rb] > 0.f);
      p.m[grow * p.num_splits + s] = empty ? -INFINITY : m_run[rb] * kLn2;
      p.l[grow * p.num_splits + s] = empty ? 0.f : l_run[rb];
    }
  }
}

template <int D, bool FP8>
static hipError_t launch_rb(const DecodeParams& p, int rb, hipStream_t st) {
  const long items = (long)p.R * p.Hkv * p.num_splits;
  dim3 grid((unsigned)((items + 3) / 4)), block(256);
  switch (rb) {
    case 1: decode_splitk_kernel<D, FP8, 1><<<grid, block, 0, st>>>(p); break;
    case 2: decode_splitk_kernel<D, FP8, 2><<<grid, block, 0, st>>>(p); break;
    case 3: decode_splitk_kernel<D, FP8, 3><<<grid, block, 0, st>>>(p); break;
    case 4: decode_splitk_kernel<D, FP8, 4><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_splitk(const DecodeParams& p, int head_dim, bool fp8,
                                int max_seqlen_q, hipStream_t st) {
  const int rows = max_seqlen_q * (p.Hq / p.Hkv);
  const int rb = (rows + 15) / 16;
  if (head_dim == 128) return fp8 ? launch_rb<128, true>(p, rb, st) : launch_rb<128, false>(p, rb, st);
  if (head_dim == 64) return fp8 ? launch_rb<64, true>(p, rb, st) : launch_rb<64, false>(p, rb, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
