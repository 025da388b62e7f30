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
};
hipError_t launch_decode_splitk(const DecodeParams& p, int head_dim, bool fp8, hipStream_t st);

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
// Zero n floats with a kernel (no memset node, so it is safe under capture).
hipError_t launch_fill_zero(float* x, long n, hipStream_t st);

}  // namespace attn
