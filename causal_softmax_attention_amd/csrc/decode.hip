// Paged split-K decode partials for 1..4 query tokens per request over a
// bf16 or per-token-scaled fp8 e4m3fn KV cache.
//
// Decode features of the prefill method (fla issue #1322, Description): an
// optional per-query-head sink (its e^sigma joins segment 0's partial), a
// sliding window (segments wholly before every row's window stream nothing)
// and the log-gate bias G_query - G_key read from a paged cache of
// cumulative gates [num_blocks, Hq, B]; and per-tensor K/V scales as an
// alternative to per-token ones (one K scale folded into the score factor,
// one V scale applied to the partial).
//
// Method (ROCm/aiter PR #6660, commit messages and "Technical details"):
// the keys of a request are split into segments; each (request, KV head,
// segment) produces (acc, m, l) partials for the query rows of the request
// that share the KV head.  Each score column is scaled by its key's K scale;
// each probability column is scaled by its key's V scale once the row sum
// has been taken, and that product is split into a bf16 high and low part
// so that PV keeps fp32 accuracy (a bf16 cache has no V scales: its P enters PV as one
// round-to-nearest bf16, as in the prefill forward); cache slots past
// seq_len never contribute (their bytes and scales may be NaN, so they are
// selected away, not multiplied by 0).  A
// query whose last visible key precedes the segment stores an empty partial
// (m = -inf, l = 0).
//
// gfx950 mapping: one workgroup per (segment, request, KV head); rows are
// (query token, head of the KV group) pairs in 16-row blocks, and a wave
// owns RBW blocks, so that the K/V conversion of a step serves all of them.
// GQA 16 with one token is a one-wave workgroup; a 4-token verify (four
// blocks) is two waves of two blocks that share every K/V tile.  The
// segment is walked 32 keys at a time through a ring of NST LDS stages:
//   * every byte a step needs (K tile, V tile, and for fp8 the per-token
//     scales) arrives by direct global->LDS copies (global_load_lds) from a
//     wave-uniform page base in SGPRs plus a fixed per-lane 32-bit offset;
//     the waves of a workgroup split the copies of a tile evenly;
//   * the copies are issued through inline asm and awaited with an explicit
//     vmcnt: the compiler, which does not track them, then neither drains
//     the ring at each LDS read nor at the barrier;
//   * page ids come through scalar loads, issued at the end of the step
//     before the one that uses them.
// K and V tiles are stored as 32 rows of D * elem bytes with 16-byte chunks
// permuted per row so that the two read patterns are free of bank conflicts
// under the bank model stated with the permutations below: MFMA operand rows
// for K (ds_read_b128) and transposed reads for V (ds_read_b64_tr_b8 for
// fp8, ds_read_b64_tr_b16 for bf16).
//   fp8 cache: K bytes become bf16 with v_cvt_scalef32_pk_bf16_fp8 (exact:
//     every e4m3 value is a bf16 value; two bytes per instruction) and
//     S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 with the bf16 query as
//     given.  (The fp8 MFMA could take the bytes directly, but it sums its
//     128 products with about 2^-13 relative error, far coarser than the
//     fp32 accumulation of the bf16 MFMA.)  V^T is converted the same way.
//   PV: O^T += V^T (P v_scale)^T with v_mfma_f32_16x16x32_bf16, once for the
//     bf16 high part of P v_scale and once for the low part (fp8 cache);
//     once with P rounded to bf16 (bf16 cache).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

// Copies of the cache (K, V and their scales).  NT: the non-temporal policy,
// for the decode and verify shapes, which read every cache byte once per
// call (measured: 64-request decode over ~1M fp8 tokens 235 -> 224 us,
// 227K-context bf16 verify 290 -> 261 us); the paged prefill, whose query
// blocks of one request read the same keys, keeps the default policy.
template <bool NT>
__device__ __forceinline__ void dma16_kv(const void* sbase, uint32_t voff, uint32_t m0) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" :: "v"(voff), "s"(sbase), "s"(m0) : "memory");
  else
    dma16(sbase, voff, m0);
}
template <bool NT>
__device__ __forceinline__ void dma4_kv(const void* sbase, uint32_t voff, uint32_t m0) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" :: "v"(voff), "s"(sbase), "s"(m0) : "memory");
  else
    dma4(sbase, voff, m0);
}

// 8 e4m3fn bytes -> 8 bf16 (exact), two bytes per instruction.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 w) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Chunk permutations of the K and V tiles (ROWB bytes per row; 16-byte
// chunk c of row r sits at chunk position c ^ swz(r)).  Bank model (measured
// on gfx950 with the bank-conflict counter): ds_read_b128 serves 32 lanes
// at a time over 512 bytes of banks, the transposed reads 32 lanes over
// 256 bytes; a read is conflict-free when those lanes hit distinct bytes
// modulo that span.
//   K, read as MFMA rows: lanes (row li of 16, group g) read logical chunk
//   g KCH + c of their row, so one instruction covers two chunks (g = 0, 1,
//   KCH apart) of 16 rows.  Rows 512 / ROWB apart share banks, and the
//   chunk pairs of those rows must land on distinct positions:
//     256-byte rows (8 rows per parity, chunks c and c + 4): bits 0, 1
//       and 3 of swz(r) distinct over the 8 rows;
//     128-byte rows (4 rows per class mod 4, chunks c and c + 2): bits 0
//       and 2 distinct over the 4 rows;
//     64-byte rows (2 rows per class mod 8, chunks 0 and 1): bit 1.
template <int ROWB>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (ROWB == 256) return ((r >> 1) & 3) | (((r >> 3) & 1) << 3);
  else if constexpr (ROWB == 128) return ((r >> 2) & 1) | (((r >> 3) & 1) << 2);
  else return ((r >> 3) & 1) << 1;
}
//   V, read transposed: fp8 lane groups read one chunk of rows
//   {4g..4g+3, 16+4g..16+4g+3}; bf16 groups read two adjacent chunks of
//   rows 4g..4g+3 (and 16+4g..).  The rows a read covers that share banks
//   (256 / ROWB apart) land on distinct positions.
template <int ROWB, bool FP8>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (FP8 && ROWB == 64) return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
  else if constexpr (FP8) return ((r >> 1) & 3) | ((r >> 2) & 4);
  else if constexpr (ROWB == 256) return (r & 7) << 1;
  else return ((r >> 1) & 3) << 1;
}

}  // namespace

// RBW: 16-row query blocks per wave; the K and V of a step are converted
// once and serve all of them.
template <int D, bool FP8, int W, int RBW, int NST, bool GATE>
__global__ __launch_bounds__(64 * W) void decode_splitk_kernel(DecodeParams p) {
  constexpr int ES = FP8 ? 1 : 2;      // bytes per cache element
  constexpr int ROWB = D * ES;         // bytes per cached token row
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;     // rows per copy instruction (64 lanes x 16 B)
  constexpr int NT = 32 * ROWB / 1024; // copy instructions per 32-row tile
  constexpr int NTW = NT / W;          // ... issued by each wave
  static_assert(NT % W == 0 && (ROWB == 64 || ROWB == 128 || ROWB == 256), "tile split");
  constexpr int KS = D / 32;           // bf16 k-steps of 32 over the head dim
  constexpr int DPG = 8 * KS;          // head-dim elements per 16-lane group
  constexpr int KCH = DPG * ES / 16;   // 16-byte K chunks per lane and key block
  constexpr int DB = D / 16;           // 16-wide output column blocks
  constexpr int TILE = 32 * ROWB;
  constexpr int SCB = FP8 ? 256 : 0;   // bytes of one scale copy (64 lanes x 4 B)
  constexpr int GTB = GATE ? 64 * 32 * 4 : 0;   // gate tile: up to 64 heads x 32 keys, fp32
  constexpr int STAGE = 2 * TILE + W * 2 * SCB + GTB;
  constexpr int LPK = 2 * NTW;         // K and V copies per step and wave (fixed;
                                       // scale and gate copies come on top)
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  constexpr bool STREAM = W * RBW <= 4;   // decode / verify shapes (not the paged prefill)
  static_assert((NST - 2) * LPK <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];

  const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;

  // ---- one segment: keys [k0, k1) of (request r, KV head kvh) for query
  // block qb; its partials go to split s (fixed-length split) or to piece
  // number s (balanced split) ----
  auto segment = [&](const int r, const int kvh, const int qb, const int k0, const int k1, const long s,
                     const bool with_sink) {
  const int L = p.seq_lens[r];
  const int qs = p.cu_q[r];
  const int qlen = p.cu_q[r + 1] - qs;
  const int G = p.Hq / p.Hkv;
  // this workgroup's rows: block qb of the request's qlen * G rows
  constexpr int RPB = 16 * W * RBW;
  const int row0 = qb * RPB;
  const int nrows = qlen * G - row0;   // rows of the block that exist (may exceed RPB)
  if (nrows <= 0) return;              // whole workgroup, before any barrier
  const int pos_min = L - qlen + row0 / G;                       // first row's position
  const int pos_max = L - qlen + (row0 + min(nrows, RPB) - 1) / G;   // last row's position
  const bool direct = p.out != nullptr;
  // A segment that starts past every row's position holds nothing for the
  // block; the reduce reads a row's segments only up to its own position.
  if (!direct && k0 > pos_max) return;
  const int k_end = min(min(L, k1), pos_max + 1);
  // first key any row of the block can see (sliding window), and where
  // this segment's streaming starts (32-key steps stay aligned; a balanced
  // piece may start and end mid-step, its other keys are masked)
  const int k_lo = p.window > 0 ? max(0, pos_min - p.window + 1) : 0;
  const int k_start = max(k0, k_lo) & ~31;
  const bool per_tensor = FP8 && p.per_tensor;
  const bool active = wave * 16 * RBW < nrows;   // wave-uniform; idle waves still copy

  // ---- copy set-up: page bases (SGPR) and fixed per-lane offsets ----
  const int bsh = p.B_shift, bmask = p.B - 1;   // page size is a power of two
  const int last_page = max(0, (L - 1) >> bsh);
  // block-table reads are wave-uniform: the constant address space makes
  // them scalar loads
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)(p.block_table + (long)r * p.max_pages);
  const long page_bytes = (long)p.Hkv * p.B * ROWB;
  const long head_bytes = (long)kvh * p.B * ROWB;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.k_cache) + head_bytes;
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.v_cache) + head_bytes;
  uint32_t voff_k[NTW], voff_v[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int r0 = (wave + W * i) * RPI;
    const int row = r0 + lane / CPR;
    voff_k[i] = (uint32_t)(((r0 & 15) + lane / CPR) * ROWB + 16 * ((lane % CPR) ^ swz_k<ROWB>(row)));
    voff_v[i] = (uint32_t)(((r0 & 15) + lane / CPR) * ROWB + 16 * ((lane % CPR) ^ swz_v<ROWB, FP8>(row)));
  }
  const uint32_t smem_lds = lds_addr(smem);

  struct Pages { int a, b; };          // pages of keys kk .. kk+15 and kk+16 .. kk+31
  auto pages_of = [&](int kk) {
    Pages pp;
    pp.a = bt[min(kk >> bsh, last_page)];
    pp.b = bt[min((kk + 16) >> bsh, last_page)];
    return pp;
  };
  // Copies of the 32-key step at kk into ring stage st.  Keys past seq_len
  // read rows of the request's last page (in range; masked later).
  auto fetch = [&](int kk, Pages pg, int st) {
    const long ra = pg.a * page_bytes + (long)(kk & bmask) * ROWB;
    const long rb = pg.b * page_bytes + (long)((kk + 16) & bmask) * ROWB;
    const uint32_t stage = smem_lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int ci = wave + W * i;
      const long ro = ci * RPI < 16 ? ra : rb;
      dma16_kv<STREAM>(kc + ro, voff_k[i], stage + ci * 1024);
      dma16_kv<STREAM>(vc + ro, voff_v[i], stage + TILE + ci * 1024);
    }
    if constexpr (FP8) {
      if (!per_tensor) {
        const int pid = (lane & 16) ? pg.b : pg.a;
        const int slot = ((kk + (lane & 16)) & bmask) + (lane & 15);
        // byte offset in unsigned 32-bit arithmetic (the host admits scale
        // arrays up to 4 GiB)
        const uint32_t so = ((((uint32_t)pid * (uint32_t)p.Hkv + (uint32_t)kvh) << bsh) + (uint32_t)slot) * 4u;
        const uint32_t sc = stage + 2 * TILE + wave * 2 * SCB;
        dma4_kv<STREAM>(p.k_scale, so, sc);
        dma4_kv<STREAM>(p.v_scale, so, sc + SCB);
      }
    }
    if constexpr (GATE) {
      // G of the group's heads at the step's keys: [G heads][32 keys], 64
      // per copy (lane l of copy c: head (64c + l) / 32, key l % 32)
      const int ngi = (G * 32 + 63) / 64;
      const uint32_t gt = stage + 2 * TILE + W * 2 * SCB;
      const int key = lane & 31;
      const int pid = (key & 16) ? pg.b : pg.a;
      const int slot = ((kk + (key & 16)) & bmask) + (key & 15);
      for (int c = wave; c < ngi; c += W) {
        const int hh = min((64 * c + lane) >> 5, G - 1);
        const uint32_t go =
            ((((uint32_t)pid * (uint32_t)p.Hq + (uint32_t)(kvh * G + hh)) << bsh) + (uint32_t)slot) * 4u;
        dma4(p.g_cache, go, gt + 256 * c);
      }
    }
  };

  // ---- prologue: first NST-1 steps in flight, then the query ----
  Pages nxt = pages_of(k_start);
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) {
    const int kk = k_start + 32 * j;
    if (kk < k_end) fetch(kk, nxt, j);
    nxt = pages_of(kk + 32);
  }

  // this lane's query rows (li of each of the wave's blocks) and Q operands
  int rho[RBW], tq[RBW], pos[RBW];
  bool rvalid[RBW];
  bf16x8 qop[RBW][KS];
  float gq2[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    rho[rb] = row0 + (wave * RBW + rb) * 16 + li;
    tq[rb] = rho[rb] / G;
    rvalid[rb] = active && tq[rb] < qlen;
    pos[rb] = L - qlen + tq[rb];                       // last key this row sees
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) +
                     ((long)(qs + min(tq[rb], qlen - 1)) * p.Hq + (long)kvh * G + rho[rb] % G) * D + g * DPG;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[rb][ks] = rvalid[rb] ? *reinterpret_cast<const bf16x8*>(qp + 8 * ks) : bf16x8{};
    // gate of the row's own position (the query side of G_query - G_key)
    gq2[rb] = 0.f;
    if constexpr (GATE) {
      const int prow = max(0, min(pos[rb], L - 1));
      const int pq = p.block_table[(long)r * p.max_pages + (prow >> bsh)];
      gq2[rb] = p.g_cache[(((long)pq * p.Hq + kvh * G + rho[rb] % G) << bsh) + (prow & bmask)] * kLog2e;
    }
  }
  // consume the loads here, while only prologue copies are in flight, so
  // that the compiler's own wait for them does not land inside the loop
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(qop[rb][ks]));
    asm volatile("" :: "v"(gq2[rb]));
  }
  // per-tensor scales: K folded into the score factor, V applied at the end
  const float qk_mul = per_tensor ? p.scale_log2 * p.k_scale[0] : p.scale_log2;
  const float v_mul = per_tensor ? p.v_scale[0] : 1.f;
  const SplitCoef coef = split_coef();
  if constexpr (FP8) {
    if (per_tensor) {
      // no scale copies: the wave's scale slots of every stage hold 1.0 (the
      // wave reads only its own slots, in order after these writes)
#pragma unroll
      for (int j = 0; j < NST; ++j) {
        float* sl = reinterpret_cast<float*>(smem + j * STAGE + 2 * TILE + wave * 2 * SCB);
        sl[lane] = 1.f;
        sl[64 + lane] = 1.f;
      }
    }
  }

  f32x4 oacc[RBW][DB];
  float m_run[RBW], l_run[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m_run[rb] = kNegBig;
    l_run[rb] = 0.f;
    if (p.sink != nullptr && with_sink) {   // the sink's mass belongs to one segment
      m_run[rb] = p.sink[kvh * G + rho[rb] % G] * kLog2e;
      l_run[rb] = 1.f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int vis_all = pos_min;         // keys up to this are visible to every row (before the window)

  auto compute = [&](int kk, int st) {
    const uint8_t* Kt = smem + st * STAGE;
    const uint8_t* Vt = Kt + TILE;
    const float* Sc = reinterpret_cast<const float*>(Kt + 2 * TILE + wave * 2 * SCB);
    const float* Gt = reinterpret_cast<const float*>(Kt + 2 * TILE + W * 2 * SCB);
    // uniform: a key past some row's position, or before some row's window
    const bool need_mask = kk + 31 > vis_all || (p.window > 0 && kk <= pos_max - p.window) || kk < k0 ||
                           kk + 31 >= k1;
    // ---- scores S^T = K Q^T (C lane: row li, keys kk+kb*16+4g+i) ----
    f32x4 sc[RBW][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 16 + li;
      i32x4 kraw[KCH];
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kraw[c] = *reinterpret_cast<const i32x4*>(Kt + row * ROWB + 16 * ((g * KCH + c) ^ swz_k<ROWB>(row)));
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) sc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kop;
        if constexpr (FP8) {
          const i32x4 w = kraw[ks / 2];
          kop = fp8x8_to_bf16x8(i32x2{w[(ks & 1) * 2], w[(ks & 1) * 2 + 1]});
        } else {
          kop = __builtin_bit_cast(bf16x8, kraw[ks]);
        }
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) sc[rb][kb] = mfma16x16x32(kop, qop[rb][ks], sc[rb][kb]);
      }
    }
    // ---- per-key K / V scale factors (shared by all rows) ----
    f32x4 ks4[2], vs4[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ks4[kb] = f32x4{1.f, 1.f, 1.f, 1.f};
      vs4[kb] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (FP8) {   // per-tensor scales: the slots hold 1.0
        ks4[kb] = *reinterpret_cast<const f32x4*>(Sc + kb * 16 + 4 * g);
        vs4[kb] = *reinterpret_cast<const f32x4*>(Sc + 64 + kb * 16 + 4 * g);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ks4[kb][i] *= qk_mul;
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 4; ++i)   // scale slots past seq_len may be NaN: select, not multiply
          vs4[kb][i] = (kk + kb * 16 + 4 * g + i < L) ? vs4[kb][i] : 0.f;
      }
    }
    bf16x8 phi[RBW], plo[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float x[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 gk4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATE) gk4 = *reinterpret_cast<const f32x4*>(Gt + (rho[rb] % G) * 32 + kb * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[kb][i] = GATE ? __builtin_fmaf(-kLog2e, gk4[i], __builtin_fmaf(sc[rb][kb][i], ks4[kb][i], gq2[rb]))
                          : sc[rb][kb][i] * ks4[kb][i];
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kk + kb * 16 + 4 * g + i;
            const bool vis = key >= k0 && key < k1 && key < L && key <= pos[rb] &&
                             (p.window <= 0 || key > pos[rb] - p.window);
            x[kb][i] = vis ? x[kb][i] : -INFINITY;
          }
      }
      // ---- online softmax (lazy rescale); P' = P * v_scale as bf16 hi + lo ----
      float mx = max3_nq(max3_nq(x[0][0], x[0][1], x[0][2]), max3_nq(x[0][3], x[1][0], x[1][1]),
                         max_nq(x[1][2], x[1][3]));
      mx = xgroup_max(mx);
      if (__any(mx > m_run[rb] + kRescaleSlack)) {
        // raise the running max only when a score passes it by more than
        // the slack, so exp2(score - max) stays below 2^8 in between
        const float m_new = max_nq(m_run[rb], mx);
        const float alpha = fast_exp2(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
        m_run[rb] = m_new;
      }
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = fast_exp2(x[kb][i] - m_run[rb]);
          const float p1 = fast_exp2(x[kb][i + 1] - m_run[rb]);
          rs += p0 + p1;
          if constexpr (FP8) {
            // hi = RNE(P'), lo = RNE(P' - hi), two columns per conversion;
            // P' - hi (exact in fp32) from one dot2 per column
            const float a = p0 * vs4[kb][i], b = p1 * vs4[kb][i + 1];
            const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
            const bf16x2 lo = __builtin_convertvector(split_lo(h, a, b, coef), bf16x2);
            phi[rb][kb * 4 + i] = h[0];
            phi[rb][kb * 4 + i + 1] = h[1];
            plo[rb][kb * 4 + i] = lo[0];
            plo[rb][kb * 4 + i + 1] = lo[1];
          } else {
            // no V scales: P itself, rounded to bf16 (RNE, unbiased, as in
            // the prefill forward); masked keys already have P = 0
            const bf16x2 h = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
            phi[rb][kb * 4 + i] = h[0];
            phi[rb][kb * 4 + i + 1] = h[1];
          }
        }
      l_run[rb] += xgroup_sum(rs);
    }
    // ---- O^T += V^T P'^T (hi and lo); V converted once for all rows ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 vop;
      if constexpr (FP8) {
        const int j = li >> 1, c = li & 1;
        const int row = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
        vop = fp8x8_to_bf16x8(lds_read_tr8(Vt + row * ROWB + 16 * (db ^ swz_v<ROWB, FP8>(row)) + 8 * c));
      } else {
        const int mm = li >> 2, c = li & 3;
        const int r0 = 4 * g + mm, r1 = 16 + 4 * g + mm, q = 2 * db + (c >> 1);
        const bf16* b0 = reinterpret_cast<const bf16*>(Vt + r0 * ROWB + 16 * (q ^ swz_v<ROWB, FP8>(r0)) + 8 * (c & 1));
        const bf16* b1 = reinterpret_cast<const bf16*>(Vt + r1 * ROWB + 16 * (q ^ swz_v<ROWB, FP8>(r1)) + 8 * (c & 1));
        vop = concat(lds_read_tr16(b0), lds_read_tr16(b1));
      }
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        oacc[rb][db] = mfma16x16x32(vop, phi[rb], oacc[rb][db]);
        if constexpr (FP8) oacc[rb][db] = mfma16x16x32(vop, plo[rb], oacc[rb][db]);
      }
    }
  };

  // ---- one step of the ring: wait for step kk, release it to the
  // workgroup, put step kk + 32 (NST-1) in flight, compute step kk ----
  auto step = [&](int kk, int st) {
    // Copies of the steps after kk that are already in flight are newer
    // than step kk's and number at least LPK each: waiting until no more
    // than that many are outstanding completes step kk's.
    if constexpr (NST == 4) {
      if (kk + 64 < k_end) wait_vm<2 * LPK>();
      else if (kk + 32 < k_end) wait_vm<LPK>();
      else wait_vm<0>();
    } else if constexpr (NST == 3) {
      if (kk + 32 < k_end) wait_vm<LPK>(); else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    if (kk + 32 > L) {
      // last step of the request: zero the V rows past seq_len that this
      // wave copied (their bytes may be NaN; P is 0 there, but 0 * NaN is not)
      uint8_t* Vt = smem + st * STAGE + TILE;
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int ci = wave + W * i;
        if (kk + ci * RPI + lane / CPR >= L)
          *reinterpret_cast<i32x4*>(Vt + ci * 1024 + 16 * lane) = i32x4{0, 0, 0, 0};
      }
    }
    if constexpr (W > 1) lds_barrier();
    const int kn = kk + 32 * (NST - 1);
    if (kn < k_end) fetch(kn, nxt, (st + NST - 1) % NST);
    if (active) compute(kk, st);
    // Page ids of the next copy: issued only now, after this step's LDS
    // reads, because a scalar load can only be awaited with lgkmcnt(0),
    // which would also wait for any LDS read issued after it.  The empty
    // asm keeps the compiler from hoisting these (invariant) loads.
    int kq = kn + 32;
    asm volatile("" : "+s"(kq) :: "memory");
    nxt = pages_of(kq);
  };

  for (int kk = k_start; kk < k_end; kk += 32 * NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      if (kk + 32 * j >= k_end) break;
      step(kk + 32 * j, j);
    }
  }
  wait_vm<0>();

  // ---- store the partials, or with a single segment the output ----
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    if (!rvalid[rb]) continue;
    const long grow = (long)(qs + tq[rb]) * p.Hq + (long)kvh * G + rho[rb] % G;
    if (direct) {
      const bool empty = !(l_run[rb] > 0.f);
      const float inv = empty ? 0.f : v_mul / l_run[rb];
      bf16* o = reinterpret_cast<bf16*>(p.out) + grow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = oacc[rb][db] * inv;
        *reinterpret_cast<bf16x4*>(o + db * 16 + 4 * g) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      }
      if (g == 0 && p.lse != nullptr)
        p.lse[grow] = empty ? -INFINITY : m_run[rb] * kLn2 + logf(l_run[rb]);
      continue;
    }
    const long slot = p.balanced ? s * p.rpu + rho[rb] : grow * p.num_splits + s;
    float* a = p.acc + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(a + db * 16 + 4 * g) = oacc[rb][db] * v_mul;
    if (g == 0) {
      const bool empty = !(l_run[rb] > 0.f);
      p.m[slot] = empty ? -INFINITY : m_run[rb] * kLn2;
      p.l[slot] = empty ? 0.f : l_run[rb];
    }
  }
  };

  if (!p.balanced) {
    int item = blockIdx.x;
    const int kvh = item % p.Hkv;
    item /= p.Hkv;
    const int r = item % p.R;
    item /= p.R;
    const int qb = item % p.nqb;
    const int s = item / p.nqb;
    segment(r, kvh, qb, s * p.split_len, (s + 1) * p.split_len, s, s == 0);
    return;
  }
  // ---- balanced split: the requests' visible keys laid end to end on one line;
  // workgroups w .. w + Hkv - 1 (dispatched together) take the same share
  // [x0, x1) of the line for the Hkv heads, so the head slices of a page are
  // read at about the same time.  Piece k of request r for head h is
  // partial (base(r) + k) * Hkv + h. ----
  const int kvh_w = blockIdx.x % p.Hkv;
  const int share = blockIdx.x / p.Hkv;
  const long total = sk_total(p.seq_lens, p.cu_q, p.window, p.R, lane);
  const long P = sk_piece_len(total, p.sk_G / p.Hkv);
  const long x0 = (long)share * P;
  if (x0 >= total) return;             // whole workgroup, before any barrier
  const long x1 = min(total, x0 + P);
  SkUnit u = sk_find(p.seq_lens, p.cu_q, p.window, p.R, P, x0, lane);
  if (u.r < 0) return;
  long piece = u.base + ((long)share - u.start / P);
  for (;;) {
    // keep the cursor in scalar registers (the copies need uniform bases)
    u.r = sk_uni(u.r);
    u.L = sk_uni(u.L);
    u.start = sk_uni(u.start);
    u.base = sk_uni(u.base);
    piece = sk_uni(piece);
    const bool first = u.start >= x0;  // this share holds the request's first key
    if (first && threadIdx.x == 0) {
      // publish the request's pieces for the reduce
      const int ui = (u.r * p.Hkv + kvh_w) * 2;
      p.unit_info[ui] = (int)u.base;
      p.unit_info[ui + 1] = sk_pieces(u.start, u.L, P);
    }
    const int lo = sk_uni(p.seq_lens[u.r] - u.L);   // the request's first visible key
    segment(sk_uni(u.r), kvh_w, 0, sk_uni(lo + (int)(max(x0, u.start) - u.start)),
            sk_uni(lo + (int)(min(x1, u.start + u.L) - u.start)), sk_uni(piece * p.Hkv + kvh_w), first);
    if (u.start + u.L >= x1) break;
    // the next request starts inside this share: its first piece is this one's
    u.base += sk_pieces(u.start, u.L, P);
    u.start += u.L;
    do {
      ++u.r;
    } while (u.r < p.R && (u.L = sk_len(p.seq_lens, p.cu_q, p.window, u.r)) == 0);
    if (u.r >= p.R) break;
    piece = u.base;
    if constexpr (W > 1) lds_barrier();   // the next piece's copies reuse the ring
  }
}

// Ring depth per launch shape.  Every stage in flight holds 32 keys of K
// and V.  Measured on one MI355X: deeper rings change neither the one-wave
// decode nor the fp8 verify (compute-bound); the bf16 verify (256-byte
// rows) gains ~3 % from four stages.
constexpr int kDecNst1 = 2, kDecNst2 = 2, kDecNst4Fp8 = 2, kDecNst4Bf16 = 4, kDecNstPrefill = 2;

// Balanced grid size: resident workgroups per CU of the instantiation that
// runs, capped for one-wave workgroups, times the CUs.  One-wave decode
// measured fastest at 3-6 workgroups per CU (fewer concurrent page streams),
// against 9 resident; two-wave verify at full residency.
constexpr int kDecBalPerCu1 = 4, kDecBalPerCu2 = 0;   // 0: no cap
// `cache` belongs to one kernel instantiation: every instantiation has the
// same function type, so the caller keeps one cache per instantiation.
template <typename K>
static int balanced_wgs(K kernel, int threads, int cap_per_cu, std::atomic<int> (&cache)[16]) {
  // per device, once per instantiation (the answer depends on nothing else)
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 16 && cache[dev].load() > 0) return cache[dev].load();
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  if (cap_per_cu > 0 && per_cu > cap_per_cu) per_cu = cap_per_cu;
  if (dev >= 0 && dev < 16) cache[dev].store(cus * per_cu);
  return cus * per_cu;
}

// Workgroups of a balanced launch of this instantiation: the resident
// workgroups (queried for the instantiation that runs), capped, in whole
// groups of Hkv (one per head).  0 on a runtime error.
template <int D, bool FP8, int W, int RBW, int NST>
static int balanced_groups_t(const DecodeParams& p) {
  const int cap = W == 1 ? kDecBalPerCu1 : kDecBalPerCu2;
  static std::atomic<int> cache_gate[16], cache_plain[16];
  const int res = p.g_cache != nullptr
                      ? balanced_wgs(decode_splitk_kernel<D, FP8, W, RBW, NST, true>, 64 * W, cap, cache_gate)
                      : balanced_wgs(decode_splitk_kernel<D, FP8, W, RBW, NST, false>, 64 * W, cap, cache_plain);
  if (res <= 0) return 0;
  int want = res < kDecodeMaxBalancedWG ? res : kDecodeMaxBalancedWG;
  want -= want % p.Hkv;
  return want > 0 ? want : p.Hkv;
}

template <int D, bool FP8, int W, int RBW, int NST>
static hipError_t launch_t(DecodeParams& p, hipStream_t st) {
  p.nqb = (p.row_blocks + W * RBW - 1) / (W * RBW);
  long items = (long)p.R * p.Hkv * p.num_splits * p.nqb;
  if (p.balanced) {
    // workgroups that stay resident together, so each share runs in one round
    p.sk_G = balanced_groups_t<D, FP8, W, RBW, NST>(p);
    if (p.sk_G <= 0) return hipErrorInvalidConfiguration;
    items = p.sk_G;
  }
  if (items > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (p.g_cache != nullptr)
    decode_splitk_kernel<D, FP8, W, RBW, NST, true><<<dim3((unsigned)items), dim3(64 * W), 0, st>>>(p);
  else
    decode_splitk_kernel<D, FP8, W, RBW, NST, false><<<dim3((unsigned)items), dim3(64 * W), 0, st>>>(p);
  return hipGetLastError();
}

// Row blocks of a (request, KV head): 1 -> one wave; 2 -> one wave holding
// both; 3 or 4 -> two waves of two blocks each; more (prefill) -> query
// blocks of 128 rows, four waves of two blocks each.  `f` is called with
// the instantiation's parameters as a tag.
template <int D, bool FP8, int W_, int RBW_, int NST_>
struct DecodeShape {
  static constexpr int W = W_, RBW = RBW_, NST = NST_;
};
template <int D, bool FP8, typename F>
static auto with_shape(int row_blocks, F f) {
  // 64-byte rows (fp8, D = 64): a 32-key tile is two copies, so at most two
  // waves share it; the prefill block keeps 128 rows as two waves of four
  if constexpr (D * (FP8 ? 1 : 2) < 128) {
    if (row_blocks > 4) return f(DecodeShape<D, FP8, 2, 4, kDecNstPrefill>{});
  } else {
    if (row_blocks > 4) return f(DecodeShape<D, FP8, 4, 2, kDecNstPrefill>{});
  }
  if (row_blocks <= 1) return f(DecodeShape<D, FP8, 1, 1, kDecNst1>{});
  if (row_blocks == 2) return f(DecodeShape<D, FP8, 1, 2, kDecNst2>{});
  return f(DecodeShape<D, FP8, 2, 2, FP8 ? kDecNst4Fp8 : kDecNst4Bf16>{});
}

template <int D, bool FP8>
static hipError_t launch_w(DecodeParams& p, hipStream_t st) {
  return with_shape<D, FP8>(p.row_blocks, [&](auto sh) {
    using S = decltype(sh);
    return launch_t<D, FP8, S::W, S::RBW, S::NST>(p, st);
  });
}

hipError_t launch_decode_splitk(DecodeParams& p, int head_dim, bool fp8, hipStream_t st) {
  if (p.row_blocks < 1) return hipErrorInvalidValue;
  if (head_dim == 128) return fp8 ? launch_w<128, true>(p, st) : launch_w<128, false>(p, st);
  if (head_dim == 64) return fp8 ? launch_w<64, true>(p, st) : launch_w<64, false>(p, st);
  return hipErrorInvalidValue;
}

int decode_balanced_groups(const DecodeParams& p, int head_dim, bool fp8) {
  if (p.row_blocks < 1) return 0;
  if (head_dim == 128 && fp8)
    return with_shape<128, true>(p.row_blocks, [&](auto sh) {
      using S = decltype(sh);
      return balanced_groups_t<128, true, S::W, S::RBW, S::NST>(p);
    });
  if (head_dim == 128)
    return with_shape<128, false>(p.row_blocks, [&](auto sh) {
      using S = decltype(sh);
      return balanced_groups_t<128, false, S::W, S::RBW, S::NST>(p);
    });
  if (head_dim == 64 && fp8)
    return with_shape<64, true>(p.row_blocks, [&](auto sh) {
      using S = decltype(sh);
      return balanced_groups_t<64, true, S::W, S::RBW, S::NST>(p);
    });
  if (head_dim == 64)
    return with_shape<64, false>(p.row_blocks, [&](auto sh) {
      using S = decltype(sh);
      return balanced_groups_t<64, false, S::W, S::RBW, S::NST>(p);
    });
  return 0;
}

}  // namespace attn
