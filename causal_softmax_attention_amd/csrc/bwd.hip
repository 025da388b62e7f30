// Backward of packed variable-length causal attention for gfx950.
//
// Method (fla issue #1322): the gradients of the Description's feature set;
// the comment of Oct 3 (sink gradient accumulated directly as an fp32 sum of
// P * (dO V^T) times the negative sink probability, reduced over queries,
// instead of through delta computed from the rounded output); the comment of
// Oct 5 (dQ fused into the dK/dV pass so each score and dP tile is computed
// once, dQ partials added into a zero-initialised fp32 buffer and converted
// to the input dtype afterwards; gate and sink partials as fp32 reductions).
//
// Three launches (plus the gate prefix scan shared with the forward):
//   bwd_pre   delta_i = sum_d fp32(O) fp32(dO); zero dq_acc, dG, dsink
//   bwd_fused one workgroup per (64-key tile, KV head, sequence); each
//             wavefront owns 16 keys and keeps K, V (B operands), K^T (for
//             dQ), dK^T and dV^T in registers, looping over the group's query
//             heads and the 32-row query tiles that see its keys:
//               S = Q K^T, dP = dO V^T             (16x16x32 MFMA)
//               P = exp2(S*c + bias - lse2), dS = P (dP - delta)
//               dV^T += dO^T P, dK^T += Q^T dS     (tr16 reads of Q, dO)
//               dQ   += dS K                       (16x16x16 MFMA, fp32 atomics)
//               dsink -= sum psink_i P_ij dP_ij,  dG_i += sum_j dS_ij,
//               dG_j -= sum_i dS_ij                (fp32)
//   bwd_post  dq = bf16(dq_acc); dg = reverse cumsum of dG per sequence
#include "common.h"
#include "kernels.h"

namespace attn {

// ---------------------------------------------------------------------------
// delta = sum_d O[row, d] * dO[row, d] in fp32 (row = token * Hq + head),
// stored head-major [Hq, T]; for the two-pass kernels also the row term
// G2 - lse * log2(e), head-major, so that a tile's rows are contiguous.
// DV/8 lanes per row, 16 bytes of O and of dO per lane, so a wave streams
// whole 256-byte rows; also zeroes the fused path's dQ accumulator and the
// gate / sink gradient accumulators.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = DV / 8;                 // lanes per row
  constexpr int RPB = 256 / LPR;              // rows per workgroup
  const int t = threadIdx.x, sub = t % LPR;
  const long row = (long)blockIdx.x * RPB + t / LPR;
  if (blockIdx.x == 0 && p.dsink_acc != nullptr)
    for (int h = t; h < p.Hq; h += 256) p.dsink_acc[h] = 0.f;
  if (row >= (long)p.T * p.Hq) return;
  // O is read once, here (non-temporal); dO is read again by both passes
  const bf16x8 o = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
      reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.o) + row * DV + 8 * sub)));
  const bf16x8 d = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(p.dO) + row * DV + 8 * sub);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)o[j] * (float)d[j];
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (sub == 0) {
    const long tok = row / p.Hq;
    const long hm = (row - tok * p.Hq) * p.T + tok;   // head-major index
    p.delta[hm] = s;
    if (p.rowt != nullptr) p.rowt[hm] = (p.G2 != nullptr ? p.G2[hm] : 0.f) - p.lse[row] * kLog2e;
    if (p.dG != nullptr) p.dG[row] = 0.f;
  }
  if (p.dq_acc != nullptr) {
    float* dqa = p.dq_acc + row * DQK;
    for (int j = sub; j < DQK / 4; j += LPR) *reinterpret_cast<f32x4*>(dqa + 4 * j) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------------------
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_fused_kernel(BwdParams p) {
  constexpr int RQ = 32;              // query rows per tile
  constexpr int BNW = 64;             // keys per workgroup (16 per wave)
  constexpr int KSQ = DQK / 32, KSV = DV / 32;
  constexpr int DBQ = DQK / 16, DBV = DV / 16;
  constexpr int QROW = DQK + 8, OROW = DV + 16;   // padded LDS strides (elements)
  __shared__ __attribute__((aligned(16))) bf16 q_lds[RQ * QROW > BNW * QROW ? RQ * QROW : BNW * QROW];
  __shared__ __attribute__((aligned(16))) bf16 do_lds[RQ * OROW];
  __shared__ __attribute__((aligned(16))) bf16 ds_lds[4][16 * RQ];
  __shared__ float lse_lds[RQ], delta_lds[RQ], gq_lds[RQ];

  const int kvh = blockIdx.x, n = blockIdx.z, ktile = blockIdx.y;
  const int seq0 = p.cu[n];
  const int L = p.cu[n + 1] - seq0;
  const int j0 = ktile * BNW;
  if (j0 >= L) return;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const int W = p.window;
  const bool gated = p.G2 != nullptr;
  const int jw = j0 + wave * 16;          // first key of this wave
  const int my_key = jw + li;             // key of this lane's score column
  const bool key_ok = my_key < L;

  // ---- K, V operands (B of S = Q K^T and dP = dO V^T): lane (key li, group g) ----
  bf16x8 kop[KSQ], vop[KSV];
  {
    const bf16* kp = reinterpret_cast<const bf16*>(p.k) + ((long)(seq0 + my_key) * p.Hkv + kvh) * DQK + 8 * g;
    const bf16* vp = reinterpret_cast<const bf16*>(p.v) + ((long)(seq0 + my_key) * p.Hkv + kvh) * DV + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) kop[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(kp + 32 * ks) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) vop[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(vp + 32 * ks) : bf16x8{};
  }
  // ---- K^T operand (B of dQ = dS K, 16x16x16): lane (d = db*16+li, keys 4g..4g+3) ----
  bf16x4 ktop[DBQ];
  {
    const bf16* kb = reinterpret_cast<const bf16*>(p.k) + ((long)seq0 * p.Hkv + kvh) * DQK;
    for (int c = tid; c < BNW * DQK / 8; c += 256) {
      const int kr = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
      i32x4 val = {0, 0, 0, 0};
      if (j0 + kr < L) val = *reinterpret_cast<const i32x4*>(kb + (long)(j0 + kr) * p.Hkv * DQK + col);
      *reinterpret_cast<i32x4*>(q_lds + kr * QROW + col) = val;
    }
    __syncthreads();
    const int mm = li >> 2, c4 = li & 3;
#pragma unroll
    for (int db = 0; db < DBQ; ++db)
      ktop[db] = lds_read_tr16(q_lds + (wave * 16 + 4 * g + mm) * QROW + db * 16 + 4 * c4);
  }

  f32x4 dk_acc[DBQ], dv_acc[DBV];
#pragma unroll
  for (int db = 0; db < DBQ; ++db) dk_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < DBV; ++db) dv_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int i_end = W > 0 ? min(L, j0 + BNW - 1 + W) : L;

  for (int hg = 0; hg < grp; ++hg) {
    const int h = kvh * grp + hg;
    const float sink2 = p.sink ? p.sink[h] * kLog2e : 0.f;
    const float gk = (gated && key_ok) ? p.G2[(long)h * p.T + seq0 + my_key] : 0.f;
    float sink_part = 0.f;   // sum over this lane's elements of psink * P * dP
    float colsum = 0.f;      // sum over rows of dS for this lane's key

    for (int i0 = j0; i0 < i_end; i0 += RQ) {
      __syncthreads();
      // ---- stage Q, dO rows i0..i0+31 of head h and their row statistics ----
      for (int c = tid; c < RQ * DQK / 8; c += 256) {
        const int rr = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        i32x4 val = {0, 0, 0, 0};
        if (i0 + rr < L)
          val = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.q) +
                                                ((long)(seq0 + i0 + rr) * p.Hq + h) * DQK + col);
        *reinterpret_cast<i32x4*>(q_lds + rr * QROW + col) = val;
      }
      for (int c = tid; c < RQ * DV / 8; c += 256) {
        const int rr = c / (DV / 8), col = (c % (DV / 8)) * 8;
        i32x4 val = {0, 0, 0, 0};
        if (i0 + rr < L)
          val = *reinterpret_cast<const i32x4*>(reinterpret_cast<const bf16*>(p.dO) +
                                                ((long)(seq0 + i0 + rr) * p.Hq + h) * DV + col);
        *reinterpret_cast<i32x4*>(do_lds + rr * OROW + col) = val;
      }
      if (tid < RQ) {
        const bool ok = i0 + tid < L;
        const long ri = (long)(seq0 + i0 + tid) * p.Hq + h;
        lse_lds[tid] = ok ? p.lse[ri] * kLog2e : 0.f;
        delta_lds[tid] = ok ? p.delta[(long)h * p.T + seq0 + i0 + tid] : 0.f;
        gq_lds[tid] = (ok && gated) ? p.G2[(long)h * p.T + seq0 + i0 + tid] : 0.f;
      }
      __syncthreads();

      // ---- skip if no (row, key) pair of this wave is visible ----
      if (jw >= L) continue;
      if (i0 + RQ - 1 < jw) continue;                       // rows all before keys
      if (W > 0 && i0 - (jw + 15) >= W) continue;           // keys all out of window

      // ---- S = Q K^T and dP = dO V^T: C lane (key li, rows rb*16+4g+i) ----
      f32x4 s[2], dp[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks)
          s[rb] = mfma16x16x32(lds_read8(q_lds + (rb * 16 + li) * QROW + ks * 32 + 8 * g), kop[ks], s[rb]);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
          dp[rb] = mfma16x16x32(lds_read8(do_lds + (rb * 16 + li) * OROW + ks * 32 + 8 * g), vop[ks], dp[rb]);
      }
      // ---- P, dS and the fp32 partial sums ----
      bf16x4 pb[2], dsb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 pv, dsv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = rb * 16 + 4 * g + i;
          const int row = i0 + rl;
          const bool vis = key_ok && row < L && my_key <= row && (W <= 0 || row - my_key < W);
          const float x = s[rb][i] * p.scale_log2 + (gq_lds[rl] - gk) - lse_lds[rl];
          const float pr = vis ? fast_exp2(x) : 0.f;
          const float pdp = pr * dp[rb][i];
          const float d = pr * (dp[rb][i] - delta_lds[rl]);
          if (p.sink) sink_part += fast_exp2(sink2 - lse_lds[rl]) * pdp;
          colsum += d;
          pv[i] = pr;
          dsv[i] = d;
        }
        pb[rb] = to_bf16x4(pv);
        dsb[rb] = to_bf16x4(dsv);
        if (gated) {
          // row sums over this wave's 16 keys: reduce across the 16 lanes of a group
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float rsum = dsv[i];
            rsum += __shfl_xor(rsum, 1);
            rsum += __shfl_xor(rsum, 2);
            rsum += __shfl_xor(rsum, 4);
            rsum += __shfl_xor(rsum, 8);
            const int row = i0 + rb * 16 + 4 * g + i;
            if (li == 0 && row < L) atomicAdd(p.dG + (long)(seq0 + row) * p.Hq + h, rsum);
          }
        }
      }
      // ---- dS^T to LDS for the dQ product (rows contiguous per key) ----
      bf16* dst = ds_lds[wave];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) *reinterpret_cast<bf16x4*>(dst + li * RQ + rb * 16 + 4 * g) = dsb[rb];

      // ---- dV^T += dO^T P and dK^T += Q^T dS (32 rows per MFMA) ----
      const bf16x8 pop = concat(pb[0], pb[1]);
      const bf16x8 dsop = concat(dsb[0], dsb[1]);
      {
        const int mm = li >> 2, c4 = li & 3;
        const bf16* o0 = do_lds + (4 * g + mm) * OROW + 4 * c4;
        const bf16* o1 = do_lds + (16 + 4 * g + mm) * OROW + 4 * c4;
#pragma unroll
        for (int db = 0; db < DBV; ++db)
          dv_acc[db] = mfma16x16x32(concat(lds_read_tr16(o0 + db * 16), lds_read_tr16(o1 + db * 16)), pop, dv_acc[db]);
        const bf16* q0 = q_lds + (4 * g + mm) * QROW + 4 * c4;
        const bf16* q1 = q_lds + (16 + 4 * g + mm) * QROW + 4 * c4;
#pragma unroll
        for (int db = 0; db < DBQ; ++db)
          dk_acc[db] = mfma16x16x32(concat(lds_read_tr16(q0 + db * 16), lds_read_tr16(q1 + db * 16)), dsop, dk_acc[db]);
      }
      // ---- dQ[rows][d] += dS K over this wave's 16 keys ----
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      {
        const int mm = li >> 2, c4 = li & 3;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const bf16x4 a = lds_read_tr16(dst + (4 * g + mm) * RQ + rb * 16 + 4 * c4);
#pragma unroll
          for (int db = 0; db < DBQ; ++db) {
            f32x4 c = mfma16x16x16(a, ktop[db], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = i0 + rb * 16 + 4 * g + i;
              if (row < L)
                atomicAdd(p.dq_acc + ((long)(seq0 + row) * p.Hq + h) * DQK + db * 16 + li, c[i] * p.scale);
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // ---- per-head partial sums: sink gradient and gate column sums ----
    if (p.sink) {
      float v = sink_part;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && v != 0.f) atomicAdd(p.dsink_acc + h, -v);
    }
    if (gated) {
      colsum += __shfl_xor(colsum, 16);
      colsum += __shfl_xor(colsum, 32);
      if (g == 0 && key_ok) atomicAdd(p.dG + (long)(seq0 + my_key) * p.Hq + h, -colsum);
    }
  }

  // ---- write dK = scale * dK^T acc, dV (lane: key li, columns db*16+4g+i) ----
  if (key_ok) {
    bf16* dkp = reinterpret_cast<bf16*>(p.dk) + ((long)(seq0 + my_key) * p.Hkv + kvh) * DQK + 4 * g;
    bf16* dvp = reinterpret_cast<bf16*>(p.dv) + ((long)(seq0 + my_key) * p.Hkv + kvh) * DV + 4 * g;
#pragma unroll
    for (int db = 0; db < DBQ; ++db) *reinterpret_cast<bf16x4*>(dkp + db * 16) = to_bf16x4(dk_acc[db] * p.scale);
#pragma unroll
    for (int db = 0; db < DBV; ++db) *reinterpret_cast<bf16x4*>(dvp + db * 16) = to_bf16x4(dv_acc[db]);
  }
}

// ---------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                             bf16* __restrict__ dq, long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = reinterpret_cast<const f32x4*>(acc)[i];
  reinterpret_cast<bf16x4*>(dq)[i] = to_bf16x4(x);
}

// dg[t, h] = sum over s >= t within t's sequence of dG[s, h] (a reverse
// scan): one workgroup per (head, sequence).  dG[t, h] = a[t, h] - b[t, h]
// (b may be null), both read at t * st_t + h * st_h (head-major partials of
// the two-pass path, token-major accumulator of the fused one).
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* __restrict__ a_,
                                                        const float* __restrict__ b_,
                                                        const int32_t* __restrict__ cu,
                                                        float* __restrict__ dg, int Hq, long st_t,
                                                        long st_h) {
  const int h = blockIdx.x, n = blockIdx.y;
  const int a = cu[n], L = cu[n + 1] - a;
  if (L <= 0) return;
  const long base = (long)a * st_t + h * st_h;
  float* out = dg + (long)a * Hq + h;
  // scan order q runs from the sequence's last token to its first
  block_scan_256(
      L,
      [&](int q) {
        const long i = base + (long)(L - 1 - q) * st_t;
        return b_ ? a_[i] - b_[i] : a_[i];
      },
      [&](int q, float v) { out[(long)(L - 1 - q) * Hq] = v; });
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* x, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

hipError_t launch_fill_zero(float* x, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_zero_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(x, n);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_fused_t(const BwdParams& p, hipStream_t st) {
  const long rows = (long)p.T * p.Hq;
  const int ktiles = (p.max_seqlen + 63) / 64;
  bwd_fused_kernel<DQK, DV><<<dim3(p.Hkv, ktiles, p.num_seqs), 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n4 = rows * DQK / 4;
  bwd_dq_convert_kernel<DQK><<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(
      p.dq_acc, reinterpret_cast<bf16*>(p.dq), n4);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.dg != nullptr) {
    gate_grad_kernel<<<dim3(p.Hq, p.num_seqs), 256, 0, st>>>(p.dG, nullptr, p.cu, p.dg, p.Hq, p.Hq, 1);
    e = hipGetLastError();
  }
  return e;
}

template <int DQK, int DV>
static hipError_t launch_bwd_t(const BwdParams& p, bool fused, hipStream_t st) {
  const long rows = (long)p.T * p.Hq;
  constexpr int RPB = 256 / (DV / 8);
  bwd_pre_kernel<DQK, DV><<<dim3((unsigned)((rows + RPB - 1) / RPB)), 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (DQK <= 128) {   // the fused-dQ path covers query/key head dims up to 128
    if (fused) return launch_fused_t<DQK, DV>(p, st);
  }
  e = launch_bwd_two_pass(p, DQK, DV, st);
  if (e != hipSuccess) return e;
  if (p.dg != nullptr) {
    gate_grad_kernel<<<dim3(p.Hq, p.num_seqs), 256, 0, st>>>(p.dGrow, p.dGcol, p.cu, p.dg, p.Hq, 1, p.T);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(const BwdParams& p, int dqk, int dv, bool fused, hipStream_t st) {
  if (p.num_seqs == 0 || p.T == 0 || p.max_seqlen == 0) {
    return hipSuccess;
  }
  switch (dqk * 1000 + dv) {
    case 64064: return launch_bwd_t<64, 64>(p, fused, st);
    case 64128: return launch_bwd_t<64, 128>(p, fused, st);
    case 64256: return launch_bwd_t<64, 256>(p, fused, st);
    case 64512: return launch_bwd_t<64, 512>(p, fused, st);
    case 128064: return launch_bwd_t<128, 64>(p, fused, st);
    case 128128: return launch_bwd_t<128, 128>(p, fused, st);
    case 128256: return launch_bwd_t<128, 256>(p, fused, st);
    case 128512: return launch_bwd_t<128, 512>(p, fused, st);
    case 256064: return launch_bwd_t<256, 64>(p, fused, st);
    case 256128: return launch_bwd_t<256, 128>(p, fused, st);
    case 256256: return launch_bwd_t<256, 256>(p, fused, st);
    case 256512: return launch_bwd_t<256, 512>(p, fused, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
