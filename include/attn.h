/*
 * attn.h -- C ABI of the MI355X (gfx950) causal softmax attention library.
 *
 * Four operations make up the hot path:
 *   attn_fwd_varlen     packed variable-length causal attention, forward
 *   attn_bwd_varlen     its gradients (dq, dk, dv, d sink, d gate)
 *   attn_decode_paged   paged single/short-query decode, split over KV segments
 *   attn_splitk_reduce  log-sum-exp merge of split-K partials
 *
 * Sources that define the operations:
 *   - fla-org/flash-linear-attention issue #1322, "[Perf] Gluon attention
 *     backend with large head dimensions": Description (the feature set:
 *     dense and packed varlen inputs, MHA/GQA/MQA, unequal q/k and v head
 *     dims up to 512, logarithmic gates, sliding windows, sink bias,
 *     gradients, packed single-query decode); comment of Oct 3 (sink
 *     gradient as a direct fp32 sum of P * (dO V^T) times the negative sink
 *     probability); comment of Oct 5 (dQ fused into the dK/dV pass through a
 *     zero-initialised fp32 buffer converted after the kernel; gate and sink
 *     partials as fp32 reductions).
 *   - ROCm/aiter PR #6660, "per-token fp8 KV scales and short-query split-K":
 *     commit messages and "Technical details" (one float32 K and V scale per
 *     cached token, [num_blocks, num_kv_heads, block_size]; K scales on the QK
 *     columns, V scales on the P columns after the row sum; slots past
 *     seq_len contribute nothing; P times the V scale split into bf16 high and
 *     low parts so that PV matches fp32; queries of at most 4 tokens run
 *     split-K; a query that ends before a segment stores an empty partial
 *     with M = -inf, weighed 0 by the reduce; NotImplementedError on paths
 *     that cannot read the scales).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * All tensor pointers are DEVICE pointers (memory the caller allocated on
 *    the GPU that `stream` belongs to).  Scalars are passed by value.
 *  * Layouts are fixed and dense (row-major, innermost dimension last, no
 *    strides); every tensor pointer must be 16-byte aligned.
 *  * bf16 means bfloat16 (1 sign, 8 exponent, 7 mantissa bits); fp8 means OCP
 *    e4m3fn (bias 7, no infinities, NaN = S.1111.111, max 448).
 *  * The caller owns every buffer, the workspace included.  The library
 *    allocates no device memory and keeps no pointer after a call returns.
 *  * Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  Results are ready when the caller synchronises.
 *  * Every argument check runs before anything is enqueued: a call that
 *    returns an error has had no effect.  attn_last_error() then gives a
 *    one-line description (per calling thread).
 *  * Packed tokens: sequence n occupies rows cu_seqlens[n] .. cu_seqlens[n+1]-1
 *    of every [T, ...] tensor; cu_seqlens is int32, non-decreasing, starts at
 *    0 and ends at total_tokens.  The library trusts these values (it cannot
 *    read device memory before launching); inconsistent values are undefined
 *    behaviour.
 *  * GQA/MQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups);
 *    Hq must be a multiple of Hkv.
 *
 * Status codes
 * ------------
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = -1,      /* malformed arguments: NULL pointer, negative or
                                 inconsistent sizes, misaligned pointer,
                                 workspace too small */
  ATTN_ERR_UNSUPPORTED = -2,  /* well-formed but not implemented: head dims,
                                 page size, KV dtype / scale combination,
                                 decode queries longer than 4 tokens */
  ATTN_ERR_HIP = -3           /* a HIP runtime call or kernel launch failed */
};

enum attn_dtype {
  ATTN_DTYPE_BF16 = 0,
  ATTN_DTYPE_FP8_E4M3FN = 1,
  ATTN_DTYPE_FP32 = 2
};

/* Human-readable name of a status code (static string). */
const char* attn_status_string(int status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* attn_last_error(void);
/* Library version string. */
const char* attn_version(void);

/* ------------------------------------------------------------------------
 * attn_fwd_varlen -- causal softmax attention over packed sequences.
 *
 * Defined by fla issue #1322, Description.  For sequence n, local query i,
 * query head h and its KV head kv = h / (Hq / Hkv):
 *   s_ij = softmax_scale * <q_i, k_j> + (G_i - G_j)       for visible j
 *   visible: j <= i, and i - j < window when window > 0
 *   G_i  = sum of g over the sequence's tokens 0..i       (gate prefix)
 *   m_i  = max(sink_h, max_j s_ij);  l_i = e^(sink_h - m_i) + sum_j e^(s_ij - m_i)
 *   o_i  = sum_j e^(s_ij - m_i) v_j / l_i;   lse_i = m_i + ln l_i
 * softmax_scale must be finite and positive (ATTN_ERR_INVALID otherwise).
 * The sink is a raw per-query-head logit with no value; without a sink,
 * sink_h = -inf; without gates, G = 0.
 *
 *   q    bf16 [total_tokens, Hq,  head_dim_qk]
 *   k    bf16 [total_tokens, Hkv, head_dim_qk]
 *   v    bf16 [total_tokens, Hkv, head_dim_v]
 *   cu_seqlens int32 [num_seqs + 1]
 *   max_seqlen  >= every sequence length (sizes the launch grid)
 *   sink fp32 [Hq] or NULL;  g fp32 [total_tokens, Hq] (log gates) or NULL
 *   o    bf16 [total_tokens, Hq, head_dim_v]   (output, round-to-nearest-even)
 *   lse  fp32 [total_tokens, Hq]               (output, natural log)
 * Supported: head_dim_qk 64, 128 or 256 with head_dim_v 64, 128, 256 or
 * 512 (every pair; other values ATTN_ERR_UNSUPPORTED).  workspace: attn_fwd_workspace_size() bytes (may be 0 / NULL
 * when that size is 0).
 * ---------------------------------------------------------------------- */
size_t attn_fwd_workspace_size(int total_tokens, int num_q_heads, int has_gate);

int attn_fwd_varlen(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                    int total_tokens, int num_q_heads, int num_kv_heads,
                    int head_dim_qk, int head_dim_v, float softmax_scale,
                    int window, const float* sink, const float* g,
                    void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * attn_bwd_varlen -- gradients of attn_fwd_varlen.
 *
 * Given dO = dL/do, with P_ij = e^(s_ij - lse_i), dP_ij = <dO_i, v_j>,
 * delta_i = sum over the row of fp32(O_i) * fp32(dO_i) (from the bf16 output,
 * as the Oct 3 comment describes for the score gradient):
 *   dS_ij  = P_ij (dP_ij - delta_i)
 *   dq_i   = scale * sum_j dS_ij k_j
 *   dk_j   = scale * sum over the group's query heads and i of dS_ij q_i
 *   dv_j   = sum over the group's query heads and i of P_ij dO_i
 *   dsink_h = -sum_i psink_i * sum_j P_ij dP_ij   (direct fp32 sum, Oct 3
 *            comment; psink_i = e^(sink_h - lse_i))
 *   dg_t   = sum over i >= t in t's sequence of
 *            (sum_j dS_ij - sum_i' dS_i'i)         (gate bias G_i - G_j)
 * Two implementations (Oct 5 comment), chosen by `flags`:
 *   0 or ATTN_BWD_DETERMINISTIC: two passes (dK/dV KV-major, then dQ
 *     Q-major); every sum is complete inside one wavefront or added in a
 *     fixed order, so results are bitwise reproducible.  For head_dim_v
 *     512, and head_dim_qk 256 with head_dim_v 128 or 256, the dK/dV pass
 *     stores dS (bf16, the rounding the dQ product uses) and the gate's fp32
 *     row sums of dS per 16-key block in the workspace, and the dQ pass reads
 *     them instead of forming S and dP again; the sink gradient is then
 *     summed per key (sum_i psink_i P_ij dP_ij) and over keys.  Other head
 *     dims, a store that would pass 32 GiB, and ATTN_BWD_RECOMPUTE_DQ: the
 *     dQ pass recomputes S and dP and sums the rows itself.
 *   ATTN_BWD_FUSED_DQ: dQ fused into the dK/dV pass, each S and dP tile
 *     computed once, dQ partials added with fp32 atomics into a zeroed fp32
 *     workspace and converted to bf16 after the kernel; gate and sink
 *     partials also through fp32 atomics, so dq, dsink and dg are not
 *     bitwise reproducible.  head_dim_qk <= 128 only (as on the page).
 * ATTN_BWD_RECOMPUTE_DQ may be added to 0 or ATTN_BWD_DETERMINISTIC.  Any
 * other flag bit, FUSED_DQ with DETERMINISTIC or RECOMPUTE_DQ, is
 * ATTN_ERR_INVALID.
 *
 *   q, k, v, cu_seqlens, sink, g, sizes: exactly as passed to the forward
 *   o    bf16 [T, Hq, head_dim_v]   the forward's output
 *   dO   bf16 [T, Hq, head_dim_v]
 *   lse  fp32 [T, Hq]               the forward's lse
 *   dq   bf16 [T, Hq,  head_dim_qk]  (output)
 *   dk   bf16 [T, Hkv, head_dim_qk]  (output)
 *   dv   bf16 [T, Hkv, head_dim_v]   (output)
 *   dsink fp32 [Hq]       output; must be NULL iff sink is NULL
 *   dg    fp32 [T, Hq]    output; must be NULL iff g is NULL
 * workspace: attn_bwd_workspace_size() bytes for the same sizes, window,
 * gate, sink and flags (the dS store needs O(Hq * T * min(window,
 * max_seqlen)) bytes: 2 per visible pair, up to twice that near the causal
 * diagonal, plus 1/8 of it for the gate's row sums).
 * ---------------------------------------------------------------------- */
enum attn_bwd_flags {
  ATTN_BWD_DETERMINISTIC = 1,  /* two-pass kernels, no atomics: bitwise
                                  reproducible (also the default path) */
  ATTN_BWD_FUSED_DQ = 2,       /* dQ fused into the dK/dV pass through fp32
                                  atomics (head_dim_qk <= 128 only) */
  ATTN_BWD_RECOMPUTE_DQ = 4     /* two-pass without the dS store: the dQ pass
                                  recomputes S and dP (less workspace) */
};

/* Workspace bytes of attn_bwd_varlen for these arguments (0 when
 * total_tokens or num_q_heads is 0). */
size_t attn_bwd_workspace_size(int total_tokens, int num_seqs, int max_seqlen,
                               int num_q_heads, int head_dim_qk, int head_dim_v,
                               int window, int has_gate, int has_sink,
                               int flags);

int attn_bwd_varlen(const void* q, const void* k, const void* v,
                    const void* o, const void* dO, const float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                    int total_tokens, int num_q_heads, int num_kv_heads,
                    int head_dim_qk, int head_dim_v, float softmax_scale,
                    int window, const float* sink, const float* g,
                    void* dq, void* dk, void* dv, float* dsink, float* dg,
                    int flags, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * attn_decode_paged -- paged decode of 1..4 new query tokens per request.
 *
 * Defined by aiter PR #6660 (commit messages, Technical details).  Request r
 * has KV length seq_lens[r] (its new tokens included) and q_len_r =
 * cu_seqlens_q[r+1] - cu_seqlens_q[r] query tokens; query t sits at position
 * seq_lens[r] - q_len_r + t and sees keys 0 .. that position.  Token j of
 * request r is stored in page block_table[r * max_pages + j / block_size],
 * slot j % block_size.  With fp8, Khat_j = k_scale[page, kv, slot] * K_j and
 * Vhat_j likewise; with bf16 the cache values are used as they are.
 *   o_t = sum_j softmax_j(softmax_scale * <q_t, Khat_j>) Vhat_j
 * Cache slots past seq_len never contribute: they may hold NaN (data or
 * scales); the kernel may copy them with the rest of their page, but masks
 * their scores, selects their scales away and zeroes their V rows.  The keys are
 * split into segments of kv_split_len tokens; each (request, KV head,
 * segment) yields partials merged by the same log-sum-exp reduce as
 * attn_splitk_reduce.  A query whose last visible key precedes a segment
 * gets an empty partial (m = -inf, weight 0).
 *
 *   q        bf16 [Tq, Hq, head_dim], Tq = cu_seqlens_q[num_requests]
 *   cu_seqlens_q int32 [num_requests + 1]; every q_len in 1 .. max_seqlen_q
 *   max_seqlen_q 1..4 (larger values: ATTN_ERR_UNSUPPORTED, "prefill")
 *   k_cache, v_cache [num_blocks, Hkv, block_size, head_dim] of kv_dtype
 *            (ATTN_DTYPE_BF16 or ATTN_DTYPE_FP8_E4M3FN)
 *   k_scale, v_scale fp32 [num_blocks, Hkv, block_size]: required for fp8,
 *            must be NULL for bf16
 *   block_table int32 [num_requests, max_pages]; seq_lens int32 [num_requests]
 *   max_seq_len >= every seq_lens[r] (sizes the split grid); at most 2^30,
 *                else ATTN_ERR_UNSUPPORTED
 *   kv_split_len 0 = library's choice, else a multiple of max(block_size, 32)
 *            and at most 8192
 *   out      bf16 [Tq, Hq, head_dim] (output)
 *   lse      fp32 [Tq, Hq] (output, natural log) or NULL
 * Supported: head_dim 64 or 128, with a bf16 or an fp8 cache;
 * block_size 16, 32, 64 or 128; max_seqlen_q * (Hq / Hkv) <= 64.
 * workspace: attn_decode_workspace_size() bytes (same arguments; SIZE_MAX
 * when the partials would pass 2^60 bytes: such calls are UNSUPPORTED); with a
 * single segment (kv_split_len >= max_seq_len) the kernel writes out and lse
 * itself, needs no workspace (size 0, workspace may be NULL) and no reduce.
 * ---------------------------------------------------------------------- */
size_t attn_decode_workspace_size(int num_requests, int max_seqlen_q,
                                  int max_seq_len, int num_q_heads,
                                  int num_kv_heads, int head_dim,
                                  int block_size, int kv_split_len);

int attn_decode_paged(const void* q, const int32_t* cu_seqlens_q,
                      int num_requests, int max_seqlen_q,
                      const void* k_cache, const void* v_cache, int kv_dtype,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int max_pages,
                      const int32_t* seq_lens, int max_seq_len,
                      int num_blocks, int block_size,
                      int num_q_heads, int num_kv_heads, int head_dim,
                      float softmax_scale, int kv_split_len,
                      void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same operation, arguments
 * and results as attn_decode_paged, without the workspace.
 *
 * The split-K partials live in a scratch array inside the library (one copy
 * per GPU, ATTN_DECODE_NOALLOC_SCRATCH_BYTES, held until the process ends);
 * its device address is looked up once per device on the first call there.
 * The call allocates and frees nothing, and calls no allocating routine.
 * The caller still passes the inputs and the outputs (out, lse).
 *
 * The partials are sized for the grid the call actually launches; a call
 * that needs more than the scratch returns ATTN_ERR_UNSUPPORTED (the
 * message names the size) and enqueues nothing.  Every call on a GPU shares
 * that GPU's scratch: calls that may overlap on one GPU (several streams,
 * or several host threads) race and must be serialised by the caller.
 * Nothing in the scratch needs to start at zero: a call reads only the
 * partials it wrote itself.
 * ------------------------------------------------------------------------ */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_decode_paged_noalloc(const void* q, const int32_t* cu_seqlens_q,
                              int num_requests, int max_seqlen_q,
                              const void* k_cache, const void* v_cache, int kv_dtype,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_table, int max_pages,
                              const int32_t* seq_lens, int max_seq_len,
                              int num_blocks, int block_size,
                              int num_q_heads, int num_kv_heads, int head_dim,
                              float softmax_scale, int kv_split_len,
                              void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * attn_decode_paged_ext -- attn_decode_paged with the decode counterparts of
 * the prefill features (fla issue #1322, Description: sink, sliding window,
 * log gate) and per-tensor KV scales (aiter PR #6660, Technical details).
 *
 * Arguments as attn_decode_paged, plus:
 *   per_tensor_scales 0: k_scale / v_scale are per-token [num_blocks, Hkv,
 *            block_size]; 1: each points to one fp32 scale for its whole
 *            cache (fp8 only)
 *   sink     fp32 [Hq] sink logits or NULL: e^sink[h] joins the softmax
 *            denominator (no value); lse includes it
 *   window   > 0: the query at position p sees keys j with p - j < window;
 *            <= 0: no window
 *   g_cache  fp32 [num_blocks, Hq, block_size] or NULL: cumulative log gate
 *            G of each cached token and query head (same paging as the KV
 *            cache); the score of key j gains G_p - G_j, with G_p read at the
 *            query's own position (its slot must hold its G)
 * The score is  softmax_scale * <q, Khat_j> + (G_p - G_j).  The sink's mass
 * is part of segment 0's partial, so attn_splitk_reduce is unchanged.
 * Per-token scale and gate arrays must each stay below 4 GiB
 * (ATTN_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */
int attn_decode_paged_ext(const void* q, const int32_t* cu_seqlens_q,
                          int num_requests, int max_seqlen_q,
                          const void* k_cache, const void* v_cache, int kv_dtype,
                          const float* k_scale, const float* v_scale,
                          int per_tensor_scales,
                          const int32_t* block_table, int max_pages,
                          const int32_t* seq_lens, int max_seq_len,
                          int num_blocks, int block_size,
                          int num_q_heads, int num_kv_heads, int head_dim,
                          float softmax_scale,
                          const float* sink, int window, const float* g_cache,
                          int kv_split_len, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * attn_prefill_paged -- paged prefill: any number of new query tokens per
 * request over the same paged bf16 / per-token fp8 cache (chunked prefill,
 * verify of more than four tokens, and mixed batches of these with decode
 * rows).
 *
 * aiter PR #6660, Technical details and third commit message: batches that
 * are not all short queries go to the other ("2d") kernel, one program per
 * (KV head, query block) over the paged cache.  The result of each row is
 * defined exactly as in attn_decode_paged_ext (positions, visibility, K and
 * V scales, sink, window, gate); only the q_len limits are lifted.
 *
 * Arguments as attn_decode_paged_ext, except:
 *   max_seqlen_q  >= 1, no upper limit (the new tokens of every request
 *            must already be in its cache: seq_lens[r] >= q_len_r)
 *   kv_split_len 0 = library's choice: one segment per query block when the
 *            query blocks alone fill the GPU (no partials, no reduce), else
 *            segments that bring the work items near 2048; or a multiple of
 *            max(block_size, 32)
 * Rows are the (token, head of the KV group) pairs of a request; a work
 * item is (segment, 128-row query block, request, KV head) and streams only
 * the keys its rows can see (causal limit and window).
 * workspace: attn_prefill_paged_workspace_size() bytes (same arguments as
 * attn_decode_workspace_size); 0 when one segment covers max_seq_len.
 * Errors: as attn_decode_paged_ext; more than 2^31 - 1 work items is
 * ATTN_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
size_t attn_prefill_paged_workspace_size(int num_requests, int max_seqlen_q,
                                         int max_seq_len, int num_q_heads,
                                         int num_kv_heads, int head_dim,
                                         int block_size, int kv_split_len);

int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q,
                       int num_requests, int max_seqlen_q,
                       const void* k_cache, const void* v_cache, int kv_dtype,
                       const float* k_scale, const float* v_scale,
                       int per_tensor_scales,
                       const int32_t* block_table, int max_pages,
                       const int32_t* seq_lens, int max_seq_len,
                       int num_blocks, int block_size,
                       int num_q_heads, int num_kv_heads, int head_dim,
                       float softmax_scale,
                       const float* sink, int window, const float* g_cache,
                       int kv_split_len, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * attn_splitk_reduce -- merge split-K partials per row (aiter PR #6660,
 * third commit message and Technical details).
 *
 * For each row r with partials s = 0..num_splits-1:
 *   M = max_s m[r,s];  w_s = e^(m[r,s] - M), or 0 when m[r,s] = -inf
 *   L = sum_s w_s l[r,s];  out[r] = sum_s w_s acc[r,s,:] / L;  lse[r] = M + ln L
 * acc and l of a split with m = -inf never enter the sums (they may be
 * read, and may hold anything, NaN included).  A row whose partials are all
 * empty gets out = 0 and lse = -inf.
 *
 *   acc fp32 [rows, num_splits, head_dim_v]  (unnormalised accumulators)
 *   m   fp32 [rows, num_splits]  (running max of natural-log logits)
 *   l   fp32 [rows, num_splits]  (sum of e^(logit - m))
 *   out [rows, head_dim_v] of out_dtype (ATTN_DTYPE_BF16 or ATTN_DTYPE_FP32)
 *   lse fp32 [rows] or NULL
 * head_dim_v: a multiple of 64, at most 512.
 * ---------------------------------------------------------------------- */
int attn_splitk_reduce(const float* acc, const float* m, const float* l,
                       int rows, int num_splits, int head_dim_v,
                       void* out, int out_dtype, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * attn_kv_cache_write_fp8 -- quantise new K/V tokens into a paged fp8 cache
 * with one scale per token and KV head (aiter PR #6660, commit messages and
 * Technical details: per-token fp8 KV scales, read back by decode).
 *
 * For each new token t and KV head h, separately for K and V:
 *   amax = max_d |x[t,h,d]|;  scale = amax / 448 (1 when amax = 0)
 *   code[d] = e4m3fn(clamp(x[t,h,d] / scale, -448, 448)), round to nearest even
 * written to page slot_mapping[t] / block_size, offset slot_mapping[t] %
 * block_size of the cache and the scales.  A negative slot (padding token)
 * or one at or past num_blocks * block_size is skipped.  Two tokens mapped
 * to the same slot leave one of them there (unspecified which).
 *
 *   k_new, v_new   bf16 [num_tokens, num_kv_heads, head_dim] (read)
 *   slot_mapping   int32 [num_tokens] (read)
 *   k_cache, v_cache  fp8 e4m3fn bytes [num_blocks, num_kv_heads, block_size,
 *                  head_dim] (written at the mapped slots only)
 *   k_scale, v_scale  fp32 [num_blocks, num_kv_heads, block_size] (same)
 * Supported: head_dim 64 or 128; block_size 16, 32, 64 or 128.
 * No workspace.  Errors as for the other entry points; nothing is launched
 * on error.
 * ---------------------------------------------------------------------- */
int attn_kv_cache_write_fp8(const void* k_new, const void* v_new,
                            const int32_t* slot_mapping, int num_tokens,
                            int num_kv_heads, int head_dim,
                            void* k_cache, void* v_cache,
                            float* k_scale, float* v_scale,
                            int num_blocks, int block_size, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
