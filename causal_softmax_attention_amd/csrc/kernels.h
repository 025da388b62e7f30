// Parameter blocks and launchers of the gfx950 kernels (internal to the
// library; the public interface is include/attn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct ReduceParams {
  const float* acc;   // [rows, num_splits, dv]
  const float* m;     // [rows, num_splits]
  const float* l;     // [rows, num_splits]
  void* out;          // [rows, dv] bf16 or fp32
  float* lse;         // [rows] or nullptr
  long rows;
  int num_splits;
  int dv;
  int out_fp32;
  // Decode rows only (else nullptr): bound the splits of each row by its
  // request's KV length.  row = token * heads + head.
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int num_requests;
  int heads;
  int split_len;
  // Balanced decode partials (see sk_* below): piece-major, rpu rows each;
  // unit_info[(r * Hkv + h) * 2 + {0, 1}] = first piece, pieces of unit (r, h).
  int balanced, rpu, Hkv;
  const int32_t* unit_info;
  // Splits (or pieces) a row is expected to hold; picks the workgroup
  // shape (more split groups for more splits).  0: num_splits.
  int splits_hint;
};
hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t st);

// Longest KV segment one decode work item walks (sizes its page-id buffer).
constexpr int kDecodeMaxSplit = 8192;

struct DecodeParams {
  const void* q;            // bf16 [Tq, Hq, D]
  const int32_t* cu_q;      // [R+1]
  const void* k_cache;      // [NB, Hkv, B, D]
  const void* v_cache;
  const float* k_scale;     // [NB, Hkv, B] (fp8 only)
  const float* v_scale;
  const int32_t* block_table;  // [R, max_pages]
  const int32_t* seq_lens;     // [R]
  float* acc;               // [Tq_max * Hq, S, D]
  float* m;                 // [Tq_max * Hq, S]
  float* l;
  int R, max_pages, Hq, Hkv, B, B_shift, split_len, num_splits;
  int row_blocks;           // 16-row query blocks per (request, KV head): ceil(max_q * G / 16)
  const float* sink;        // [Hq] sink logits or nullptr
  const float* g_cache;     // [NB, Hq, B] cumulative log gates or nullptr
  int window;               // sliding window (<= 0: none)
  int per_tensor;           // fp8 with one K and one V scale (k_scale[0], v_scale[0])
  float scale_log2;         // softmax_scale * log2(e)
  // Single segment (num_splits == 1): the kernel writes the normalised
  // output bf16 [Tq, Hq, D] and lse [Tq, Hq] (may be nullptr) itself and
  // acc / m / l are unused; nullptr otherwise.
  void* out;
  float* lse;
  int nqb;                  // query blocks per (request, KV head); set by the launcher
  // Balanced split (decode without a window): every workgroup takes an equal
  // share of all keys (see sk_* below); partials are indexed by piece:
  // acc [pieces, rpu, D], m / l [pieces, rpu] with rpu = rows per
  // (request, KV head).  sk_G (workgroups) is set by the launcher.
  int balanced;
  int rpu;
  int sk_G;
  int32_t* unit_info;       // [R * Hkv][2]: first piece and piece count of each unit (written here)
};
// Sets p.nqb and, for a balanced launch, p.sk_G.
hipError_t launch_decode_splitk(DecodeParams& p, int head_dim, bool fp8, hipStream_t st);
// Paged prefill as a pipelined 64-key tile loop (prefill_paged.hip): bf16 or
// fp8 cache (per-token or per-tensor scales), sink, window and gate; one
// segment per query tile (output written directly), softmax_scale > 0.
bool paged_pipe_supported(const DecodeParams& p, int head_dim, bool fp8, float softmax_scale);
hipError_t launch_paged_pipe(const DecodeParams& p, int head_dim, bool fp8, int max_q, hipStream_t st);
// The workgroup count (p.sk_G) a balanced launch with these parameters
// would use (host side; 0 on a runtime error).
int decode_balanced_groups(const DecodeParams& p, int head_dim, bool fp8);
// Workgroups of a balanced launch never exceed this (sizes the partials).
constexpr int kDecodeMaxBalancedWG = 4096;

// ---------------------------------------------------------------------------
// Balanced split of a decode call.  Units (requests, or (request, head)
// pairs) are laid end to end on one line; share w of n takes the keys
// [w P, (w + 1) P) of the line, P = ceil(total / n) rounded up to 32.  Each
// overlap of a unit with a share is one piece; pieces are numbered unit by
// unit, so unit u's pieces are base(u) .. base(u) + n(u) - 1.  Every wave
// computes the plan itself from seq_lens (no extra launch).
// Line positions stay below 2^31 (the host enables the balanced split only
// then), so the divisions are 32-bit.
__device__ __forceinline__ int sk_pieces(long c, int L, long P) {
  const unsigned cu = (unsigned)c, Pu = (unsigned)P;
  return L > 0 ? (int)((cu + (unsigned)L - 1u) / Pu - cu / Pu + 1u) : 0;
}
__device__ __forceinline__ long wave_incl_scan(long v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}
// wave-uniform copies (scalar registers) of values every lane holds alike
__device__ __forceinline__ int sk_uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long sk_uni(long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(v & 0xffffffffL));
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long)v >> 32));
  return (long)(((unsigned long)hi << 32) | lo);
}
// Keys of request i on the line: those its queries can see (all of them
// without a window; from the first query's window start with one).
__device__ __forceinline__ int sk_len(const int32_t* seq_lens, const int32_t* cu, int window, int i) {
  const int L = seq_lens[i];
  if (window <= 0) return L;
  const int lo = L - (cu[i + 1] - cu[i]) - window + 1;
  return lo > 0 ? L - lo : L;
}
__device__ __forceinline__ long sk_total(const int32_t* seq_lens, const int32_t* cu, int window, int R,
                                         int lane) {
  long t = 0;
  for (int c = 0; c < R; c += 64) t += (c + lane < R) ? sk_len(seq_lens, cu, window, c + lane) : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
  return sk_uni(t);
}
__device__ __forceinline__ long sk_piece_len(long total, int nshares) {
  const long P = (total + nshares - 1) / nshares;
  return P < 32 ? 32 : (P + 31) / 32 * 32;
}
struct SkUnit {
  int r, kvh, L;      // request, (unused), keys on the line
  long start, base;   // first line position of the request; its first piece's number
};
// The unit that holds line position x (by_unit: the unit (r_want, kvh_want)
// instead).  Uniform across the wave.
// The request whose keys hold line position x (uniform across the wave).
__device__ __forceinline__ SkUnit sk_find(const int32_t* seq_lens, const int32_t* cu, int window, int R,
                                          long P, long x, int lane) {
  long S = 0, B = 0;   // keys and pieces of the requests before this chunk
  SkUnit u{-1, 0, 0, 0, 0};
  for (int c = 0; c < R; c += 64) {
    const int i = c + lane;
    const int Li = i < R ? sk_len(seq_lens, cu, window, i) : 0;
    const long incl = wave_incl_scan(Li, lane);
    const long rs = S + incl - Li;   // first line position of request i
    const int Ni = sk_pieces(rs, Li, P);
    const long Nincl = wave_incl_scan(Ni, lane);
    const bool hit = i < R && Li > 0 && rs <= x && x < rs + Li;
    const unsigned long long m = __ballot(hit);
    if (m != 0) {
      const int j = __builtin_ctzll(m);
      u.r = sk_uni(c + j);
      u.L = sk_uni(__shfl(Li, j, 64));
      u.start = sk_uni(__shfl(rs, j, 64));
      u.base = sk_uni(B + __shfl(Nincl, j, 64) - __shfl(Ni, j, 64));
      return u;
    }
    S += __shfl(incl, 63, 64);
    B += __shfl(Nincl, 63, 64);
  }
  return u;
}

struct KvWriteParams {
  const void* k_new;        // bf16 [N, Hkv, D]
  const void* v_new;
  const int32_t* slot_mapping;  // [N]: page * B + offset, < 0 to skip
  void* k_cache;            // fp8 bytes [NB, Hkv, B, D]
  void* v_cache;
  float* k_scale;           // [NB, Hkv, B]
  float* v_scale;
  int N, Hkv, NB, B;
};
hipError_t launch_kv_cache_write_fp8(const KvWriteParams& p, int head_dim, hipStream_t st);

struct FwdParams {
  const void* q;            // bf16 [T, Hq, DQK]
  const void* k;            // bf16 [T, Hkv, DQK]
  const void* v;            // bf16 [T, Hkv, DV]
  const int32_t* cu;        // [N+1]
  const float* sink;        // [Hq] or nullptr
  const float* g;           // [T, Hq] log gates or nullptr
  float* G2;                // [Hq, T] workspace: gate prefix * log2(e) (head-major)
  void* o;                  // bf16 [T, Hq, DV]
  float* lse;               // [T, Hq]
  int num_seqs, max_seqlen, T, Hq, Hkv, window;
  float scale_log2;         // softmax_scale * log2(e)
};
hipError_t launch_gate_prefix(const float* g, const int32_t* cu, float* G2,
                              int num_seqs, int T, int Hq, hipStream_t st);
hipError_t launch_fwd(const FwdParams& p, int dqk, int dv, hipStream_t st);
hipError_t launch_fwd_wide(const FwdParams& p, int dqk, int dv, hipStream_t st);
hipError_t launch_fwd_large_qk64(const FwdParams& p, int dv, hipStream_t st);
hipError_t launch_fwd_large_qk128(const FwdParams& p, int dv, hipStream_t st);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;         // [T, Hq]
  const int32_t* cu;
  const float* sink;
  const float* G2;          // [Hq, T] gate prefix * log2(e) (head-major) or nullptr
  float* delta;             // [Hq, T] workspace (head-major)
  float* rowt;              // [Hq, T] workspace, two-pass only: G2 - lse * log2(e) (head-major)
  float* dq_acc;            // [T, Hq, DQK] fp32 workspace (fused dQ only)
  float* dG;                // [T, Hq] fp32 (fused: row minus column sums, by atomics)
  float* dGrow;             // [Hq, T] fp32 (two-pass: row sums of dS, stored; head-major)
  float* dGcol;             // [Hq, T] fp32 (two-pass: column sums of dS, stored; head-major)
  float* sink_rows;         // [Hq, T] fp32 (two-pass: psink_i * sum_j P_ij dP_ij; head-major)
  float* dsink_acc;         // [Hq] fp32 (the dsink output itself)
  // two-pass with a dS store (layout in bwd_ds.h); ds == nullptr: dQ pass recomputes S, dP
  void* ds;                 // bf16 dS tiles
  float* ds_rows;           // fp32 row sums of dS per tile (gate) or nullptr
  float* psink;             // [Hq, T] psink_i = e^(sink_h - lse_i) (with a sink) or nullptr
  long ds_nrt;              // row tiles of the layout
  int ds_nslot;             // key-block slots per row tile
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  int num_seqs, max_seqlen, T, Hq, Hkv, window;
  float scale;              // softmax_scale
  float scale_log2;
};
// Fused dQ (fp32 atomics) or deterministic two-pass backward, plus the
// shared pre/post kernels.
hipError_t launch_bwd(const BwdParams& p, int dqk, int dv, bool fused, hipStream_t st);
hipError_t launch_bwd_two_pass(const BwdParams& p, int dqk, int dv, hipStream_t st);
hipError_t launch_bwd_two_pass_qk64(const BwdParams& p, int dv, hipStream_t st);
hipError_t launch_bwd_two_pass_qk128(const BwdParams& p, int dv, hipStream_t st);
hipError_t launch_bwd_two_pass_qk256(const BwdParams& p, int dv, hipStream_t st);
hipError_t launch_sink_reduce(const BwdParams& p, hipStream_t st);
hipError_t launch_dkdv_large(const BwdParams& p, int dqk, int dv, hipStream_t st);
hipError_t launch_dq_large(const BwdParams& p, int dqk, int dv, hipStream_t st);
// Zero n floats with a kernel (no memset node, so it is safe under capture).
hipError_t launch_fill_zero(float* x, long n, hipStream_t st);

}  // namespace attn
