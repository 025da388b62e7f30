// C ABI of the attention library: argument validation, workspace layout and
// launch of the gfx950 kernels.  Every check runs before the first launch,
// so a call that returns an error has enqueued nothing.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/attn.h"
#include "bwd_ds.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(ATTN_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)
#define REQ_PTR(p, align)                                                               \
  do {                                                                                  \
    if ((p) == nullptr) return fail(ATTN_ERR_INVALID, "%s is NULL", #p);                \
    if (!aligned((p), (align)))                                                         \
      return fail(ATTN_ERR_INVALID, "%s is not %d-byte aligned", #p, (int)(align));     \
  } while (0)

bool fwd_dims_supported(int dqk, int dv) {
  return (dqk == 64 || dqk == 128 || dqk == 256) && (dv == 64 || dv == 128 || dv == 256 || dv == 512);
}

int check_prefill_common(const void* q, const void* k, const void* v, const int32_t* cu, int num_seqs,
                         int max_seqlen, int T, int Hq, int Hkv, int dqk, int dv, float scale) {
  REQUIRE(num_seqs >= 0 && T >= 0 && max_seqlen >= 0, ATTN_ERR_INVALID,
          "negative size (num_seqs=%d total_tokens=%d max_seqlen=%d)", num_seqs, T, max_seqlen);
  REQUIRE(Hq >= 1 && Hkv >= 1, ATTN_ERR_INVALID, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  REQUIRE(Hq % Hkv == 0, ATTN_ERR_INVALID, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", Hq, Hkv);
  REQUIRE(fwd_dims_supported(dqk, dv), ATTN_ERR_UNSUPPORTED,
          "head dims (d_qk=%d, d_v=%d) not supported; supported: d_qk in {64, 128, 256}, d_v in {64, 128, 256, 512}",
          dqk, dv);
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_ERR_INVALID,
          "softmax_scale must be finite and positive (got %g)", (double)scale);
  REQUIRE(num_seqs <= 65535, ATTN_ERR_UNSUPPORTED, "num_seqs %d exceeds 65535", num_seqs);
  REQUIRE(Hq <= 65535, ATTN_ERR_UNSUPPORTED, "num_q_heads %d exceeds 65535", Hq);
  if (num_seqs > 0 && T > 0) {
    REQUIRE(max_seqlen >= 1 && max_seqlen <= T, ATTN_ERR_INVALID,
            "max_seqlen %d must be in [1, total_tokens=%d]", max_seqlen, T);
    REQUIRE(max_seqlen <= 65535 * 16, ATTN_ERR_UNSUPPORTED, "max_seqlen %d too large", max_seqlen);
    REQ_PTR(q, 16);
    REQ_PTR(k, 16);
    REQ_PTR(v, 16);
    REQ_PTR(cu, 4);
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

const char* attn_version(void) { return "attn-mi355x 0.1 (gfx950)"; }

// ---------------------------------------------------------------------------
size_t attn_fwd_workspace_size(int total_tokens, int num_q_heads, int has_gate) {
  if (!has_gate || total_tokens <= 0 || num_q_heads <= 0) return 0;
  return round_up((size_t)total_tokens * num_q_heads * sizeof(float));
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    int num_seqs, int max_seqlen, int total_tokens, int num_q_heads,
                    int num_kv_heads, int head_dim_qk, int head_dim_v, float softmax_scale,
                    int window, const float* sink, const float* g, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prefill_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, total_tokens, num_q_heads,
                                num_kv_heads, head_dim_qk, head_dim_v, softmax_scale);
  if (st != ATTN_OK) return st;
  if (num_seqs == 0 || total_tokens == 0) return ok();
  REQ_PTR(o, 16);
  REQ_PTR(lse, 4);
  if (sink) REQ_PTR(sink, 4);
  if (g) REQ_PTR(g, 4);
  const size_t need = attn_fwd_workspace_size(total_tokens, num_q_heads, g != nullptr);
  REQUIRE(workspace_bytes >= need, ATTN_ERR_INVALID, "workspace too small: %zu < %zu bytes",
          workspace_bytes, need);
  if (need) REQ_PTR(workspace, 256);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.cu = cu_seqlens; p.sink = sink; p.g = g;
  p.G2 = g ? reinterpret_cast<float*>(workspace) : nullptr;
  p.o = o; p.lse = lse;
  p.num_seqs = num_seqs; p.max_seqlen = max_seqlen; p.T = total_tokens;
  p.Hq = num_q_heads; p.Hkv = num_kv_heads; p.window = window;
  p.scale_log2 = softmax_scale * attn::kLog2e;
  hipError_t e;
  if (g) {
    e = attn::launch_gate_prefix(g, cu_seqlens, p.G2, num_seqs, total_tokens, num_q_heads, s);
    if (e != hipSuccess) return hip_fail(e, "gate prefix launch");
  }
  e = attn::launch_fwd(p, head_dim_qk, head_dim_v, s);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

// ---------------------------------------------------------------------------
namespace {
struct BwdLayout {
  size_t delta, G2, dq_acc, dG, dGrow, dGcol, sink_rows, rowt, ds, ds_rows, psink, total;
  bool fused, store_ds;
  long ds_nrt;
  int ds_nslot;
};
// Largest dS store the two-pass backward takes by itself (bf16 tiles plus
// the gate's row partials); beyond it the dQ pass recomputes S and dP.
constexpr size_t kBwdDsMaxBytes = size_t(32) << 30;
// The dS store pays where recomputing S and dP in the dQ pass costs more than
// writing and reading 2 bytes per pair.  Measured on one MI355X (whole
// backward, causal, with or without it): d 256 x 512 on 4 x 8192 tokens
// 13.9 -> 10.5 ms; 2 x 4096 tokens: 128 x 512 2.04 -> 1.78 ms, 64 x 512
// 1.72 -> 1.67 ms, 256 x 128 1.19 -> 1.17 ms, 128 x 256 unchanged; 8
// sequences, window 1024, 128 x 128: 0.87 -> 0.93 ms (slower).  Pairs not
// measured recompute.
bool bwd_ds_pays(int dqk, int dv) { return dv == 512 || (dqk == 256 && dv >= 128); }
// Which backward runs: the fused-dQ kernel (fp32 atomics; the pages keep it
// to head dims up to 128) only when asked for, the two-pass kernels
// otherwise (faster on this GPU, and deterministic).
bool bwd_uses_fused(int dqk, int flags) {
  return (flags & ATTN_BWD_FUSED_DQ) && !(flags & ATTN_BWD_DETERMINISTIC) && dqk <= 128;
}
BwdLayout bwd_layout(int T, int num_seqs, int max_seqlen, int Hq, int dqk, int dv, int window, int has_gate,
                     int has_sink, int flags) {
  BwdLayout L{};
  const size_t rows = (size_t)(T > 0 ? T : 0) * (Hq > 0 ? Hq : 0);
  const size_t r4 = round_up(rows * sizeof(float));
  L.fused = bwd_uses_fused(dqk, flags);
  if (!L.fused && !(flags & ATTN_BWD_RECOMPUTE_DQ) && bwd_ds_pays(dqk, dv) && T > 0 && Hq > 0 && num_seqs > 0 &&
      max_seqlen > 0) {
    L.ds_nrt = attn::ds_row_tiles(T, num_seqs);
    L.ds_nslot = attn::ds_slots(max_seqlen, window);
    // in floating point first: the exact product can pass 2^64 for extreme sizes
    const double per_tile = attn::kDsTileBytes + (has_gate ? attn::kDsRows * sizeof(float) : 0);
    L.store_ds = (double)Hq * (double)L.ds_nrt * (double)L.ds_nslot * per_tile <= (double)kBwdDsMaxBytes;
  }
  size_t off = 0;
  L.delta = off; off += r4;
  L.G2 = off; if (has_gate) off += r4;
  L.rowt = off; off += r4;
  if (L.fused) {
    L.dq_acc = off; off += round_up(rows * (size_t)(dqk > 0 ? dqk : 0) * sizeof(float));
    L.dG = off; if (has_gate) off += r4;
  } else {
    L.dGrow = off; if (has_gate) off += r4;
    L.dGcol = off; if (has_gate) off += r4;
    L.sink_rows = off; if (has_sink) off += r4;
    if (L.store_ds) {
      const size_t tiles = (size_t)Hq * (size_t)L.ds_nrt * (size_t)L.ds_nslot;
      L.ds = off; off += round_up(tiles * attn::kDsTileBytes);
      L.ds_rows = off; if (has_gate) off += round_up(tiles * attn::kDsRows * sizeof(float));
      L.psink = off; if (has_sink) off += r4;
    }
  }
  L.total = off;
  return L;
}
}  // namespace

size_t attn_bwd_workspace_size(int total_tokens, int num_seqs, int max_seqlen, int num_q_heads,
                               int head_dim_qk, int head_dim_v, int window, int has_gate, int has_sink,
                               int flags) {
  if (total_tokens <= 0 || num_q_heads <= 0) return 0;
  return bwd_layout(total_tokens, num_seqs, max_seqlen, num_q_heads, head_dim_qk, head_dim_v, window, has_gate,
                    has_sink, flags)
      .total;
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                    int total_tokens, int num_q_heads, int num_kv_heads, int head_dim_qk,
                    int head_dim_v, float softmax_scale, int window, const float* sink,
                    const float* g, void* dq, void* dk, void* dv, float* dsink, float* dg, int flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prefill_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, total_tokens, num_q_heads,
                                num_kv_heads, head_dim_qk, head_dim_v, softmax_scale);
  if (st != ATTN_OK) return st;
  REQUIRE((sink == nullptr) == (dsink == nullptr), ATTN_ERR_INVALID,
          "dsink must be given exactly when sink is given");
  REQUIRE((g == nullptr) == (dg == nullptr), ATTN_ERR_INVALID, "dg must be given exactly when g is given");
  REQUIRE((flags & ~(ATTN_BWD_DETERMINISTIC | ATTN_BWD_FUSED_DQ | ATTN_BWD_RECOMPUTE_DQ)) == 0, ATTN_ERR_INVALID,
          "unknown flags 0x%x", flags);
  REQUIRE(!((flags & ATTN_BWD_FUSED_DQ) && (flags & ATTN_BWD_RECOMPUTE_DQ)), ATTN_ERR_INVALID,
          "ATTN_BWD_RECOMPUTE_DQ belongs to the two-pass backward, not ATTN_BWD_FUSED_DQ");
  REQUIRE(!((flags & ATTN_BWD_FUSED_DQ) && (flags & ATTN_BWD_DETERMINISTIC)), ATTN_ERR_INVALID,
          "ATTN_BWD_FUSED_DQ and ATTN_BWD_DETERMINISTIC exclude each other");
  REQUIRE(!((flags & ATTN_BWD_FUSED_DQ) && head_dim_qk > 128), ATTN_ERR_UNSUPPORTED,
          "the fused-dQ backward covers head_dim_qk <= 128 (got %d)", head_dim_qk);
  if (num_seqs == 0 || total_tokens == 0) {
    // Nothing to differentiate; a sink gradient over no tokens is zero.
    if (dsink != nullptr && num_q_heads > 0) {
      REQ_PTR(dsink, 4);
      hipError_t e = attn::launch_fill_zero(dsink, num_q_heads, reinterpret_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, "dsink clear");
    }
    return ok();
  }
  REQ_PTR(o, 16);
  REQ_PTR(dO, 16);
  REQ_PTR(lse, 4);
  REQ_PTR(dq, 16);
  REQ_PTR(dk, 16);
  REQ_PTR(dv, 16);
  if (sink) { REQ_PTR(sink, 4); REQ_PTR(dsink, 4); }
  if (g) { REQ_PTR(g, 4); REQ_PTR(dg, 4); }
  const BwdLayout lay = bwd_layout(total_tokens, num_seqs, max_seqlen, num_q_heads, head_dim_qk, head_dim_v,
                                   window, g != nullptr, sink != nullptr, flags);
  REQUIRE(workspace_bytes >= lay.total, ATTN_ERR_INVALID, "workspace too small: %zu < %zu bytes",
          workspace_bytes, lay.total);
  REQ_PTR(workspace, 256);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  attn::BwdParams p{};
  float* G2 = g ? reinterpret_cast<float*>(ws + lay.G2) : nullptr;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dO = dO; p.lse = lse; p.cu = cu_seqlens; p.sink = sink;
  p.G2 = G2;
  p.delta = reinterpret_cast<float*>(ws + lay.delta);
  if (lay.fused) {
    p.dq_acc = reinterpret_cast<float*>(ws + lay.dq_acc);
    p.dG = g ? reinterpret_cast<float*>(ws + lay.dG) : nullptr;
  } else {
    p.dGrow = g ? reinterpret_cast<float*>(ws + lay.dGrow) : nullptr;
    p.dGcol = g ? reinterpret_cast<float*>(ws + lay.dGcol) : nullptr;
    p.sink_rows = sink ? reinterpret_cast<float*>(ws + lay.sink_rows) : nullptr;
    if (lay.store_ds) {
      p.ds = ws + lay.ds;
      p.ds_rows = g ? reinterpret_cast<float*>(ws + lay.ds_rows) : nullptr;
      p.psink = sink ? reinterpret_cast<float*>(ws + lay.psink) : nullptr;
      p.ds_nrt = lay.ds_nrt;
      p.ds_nslot = lay.ds_nslot;
    }
  }
  p.rowt = reinterpret_cast<float*>(ws + lay.rowt);
  p.dsink_acc = dsink;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg;
  p.num_seqs = num_seqs; p.max_seqlen = max_seqlen; p.T = total_tokens;
  p.Hq = num_q_heads; p.Hkv = num_kv_heads; p.window = window;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * attn::kLog2e;
  hipError_t e;
  if (g) {
    e = attn::launch_gate_prefix(g, cu_seqlens, G2, num_seqs, total_tokens, num_q_heads, s);
    if (e != hipSuccess) return hip_fail(e, "gate prefix launch");
  }
  e = attn::launch_bwd(p, head_dim_qk, head_dim_v, lay.fused, s);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

// ---------------------------------------------------------------------------
namespace {
int choose_split_len(int R, int Hkv, int max_seq_len, int B) {
  // Aim at ~2048 wavefront work items: long enough segments to amortise the
  // partial traffic, enough of them to keep every SIMD streaming.
  const double est_tokens = (double)R * max_seq_len * 0.5;
  const double want = est_tokens * Hkv / 2048.0;
  int sl = 256;
  while (sl < want && sl < attn::kDecodeMaxSplit) sl *= 2;
  const int unit = B > 32 ? B : 32;
  if (sl < unit) sl = unit;
  return sl;
}

// Query blocks per (request, KV head) of the launch: one block of up to 64
// rows for short queries, blocks of 128 rows beyond that.
int query_blocks(int max_q, int Hq, int Hkv) {
  const long rows = (long)max_q * (Hq / Hkv);
  return rows <= 64 ? 1 : (int)((rows + 127) / 128);
}

// Paged prefill: enough query blocks already fill the chip, so one segment
// per block (no partials, no reduce); otherwise segments that bring the
// work items near 2048.
int choose_split_len_prefill(int R, int Hkv, int nqb, int max_seq_len, int B) {
  const int unit = B > 32 ? B : 32;
  const long items = (long)R * Hkv * nqb;
  const long whole = ((long)max_seq_len + unit - 1) / unit * unit;
  if (items >= 1024) return (int)std::min<long>(whole, 1L << 30);
  const long want = (2048 + items - 1) / items;
  long sl = ((max_seq_len + want - 1) / want + unit - 1) / unit * unit;
  sl = std::max<long>(sl, std::max(256, unit));
  return (int)std::min(sl, whole);
}

struct DecLayout {
  size_t acc, m, l, units, total;
  int split_len, num_splits;
};
// balanced_groups > 0: the call is known to run the balanced split with
// that many workgroups, and the partials are sized for exactly its pieces
// ((groups + R * Hkv) per row of a unit); 0: room for either split, with
// the largest balanced grid.
DecLayout dec_layout(int R, int max_q, int max_seq_len, int Hq, int Hkv, int D, int B, int split_len,
                     bool prefill = false, int balanced_groups = 0) {
  DecLayout L{};
  L.split_len = split_len > 0 ? split_len
                : prefill ? choose_split_len_prefill(R, Hkv, query_blocks(max_q, Hq, Hkv), max_seq_len, B)
                          : choose_split_len(R, Hkv, max_seq_len, B);
  L.num_splits = (int)(((long)max_seq_len + L.split_len - 1) / L.split_len);
  if (L.num_splits == 1) return L;     // single segment: the kernel writes the output
  // partial slots: rows x splits (fixed-length split), and for a decode with
  // the library's split also pieces x rows-per-unit (balanced split, used
  // when there is no window); room for the larger
  // (sizes past 2^60 bytes, where the exact products could wrap, are
  // reported as SIZE_MAX: no workspace can hold them)
  const double est = ((double)R * max_q * Hq * std::max(L.num_splits, 1) + attn::kDecodeMaxBalancedWG * 64.0) *
                     ((double)D + 2) * sizeof(float);
  if (est > 1.1529215e18) {
    L.total = SIZE_MAX;
    return L;
  }
  size_t slots = balanced_groups > 0 ? 0 : (size_t)R * max_q * Hq * L.num_splits;
  if (!prefill && split_len == 0) {
    const size_t groups = balanced_groups > 0 ? (size_t)balanced_groups : (size_t)attn::kDecodeMaxBalancedWG;
    const size_t pieces = groups + (size_t)R * Hkv;
    slots = std::max(slots, pieces * (size_t)max_q * (Hq / Hkv));
  }
  size_t off = 0;
  L.acc = off; off += round_up(slots * (size_t)D * sizeof(float));
  L.m = off; off += round_up(slots * sizeof(float));
  L.l = off; off += round_up(slots * sizeof(float));
  L.units = off; off += round_up((size_t)R * Hkv * 2 * sizeof(int32_t));
  L.total = off;
  return L;
}
}  // namespace

size_t attn_decode_workspace_size(int num_requests, int max_seqlen_q, int max_seq_len, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int kv_split_len) {
  if (num_requests <= 0 || max_seqlen_q <= 0 || max_seq_len <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || kv_split_len < 0)
    return 0;
  return dec_layout(num_requests, max_seqlen_q, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                    block_size, kv_split_len).total;
}

int attn_decode_paged(const void* q, const int32_t* cu_seqlens_q, int num_requests, int max_seqlen_q,
                      const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                      const float* v_scale, const int32_t* block_table, int max_pages,
                      const int32_t* seq_lens, int max_seq_len, int num_blocks, int block_size,
                      int num_q_heads, int num_kv_heads, int head_dim, float softmax_scale,
                      int kv_split_len, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attn_decode_paged_ext(q, cu_seqlens_q, num_requests, max_seqlen_q, k_cache, v_cache, kv_dtype,
                               k_scale, v_scale, 0, block_table, max_pages, seq_lens, max_seq_len,
                               num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, softmax_scale,
                               nullptr, 0, nullptr, kv_split_len, out, lse, workspace, workspace_bytes,
                               stream);
}

namespace {
void* scratch_on_current_device(int* status);

// noalloc: the partials go to the library's own scratch array on the current
// device (the allocation-free decode) instead of the caller's workspace.
int paged_attention(bool prefill, const void* q, const int32_t* cu_seqlens_q, int num_requests,
                    int max_seqlen_q, const void* k_cache, const void* v_cache, int kv_dtype,
                    const float* k_scale, const float* v_scale, int per_tensor_scales,
                    const int32_t* block_table, int max_pages, const int32_t* seq_lens, int max_seq_len,
                    int num_blocks, int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                    float softmax_scale, const float* sink, int window, const float* g_cache,
                    int kv_split_len, void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream, bool noalloc = false) {
  REQUIRE(num_requests >= 0, ATTN_ERR_INVALID, "num_requests %d is negative", num_requests);
  REQUIRE(max_seqlen_q >= 1, ATTN_ERR_INVALID, "max_seqlen_q %d must be >= 1", max_seqlen_q);
  REQUIRE(prefill || max_seqlen_q <= 4, ATTN_ERR_UNSUPPORTED,
          "max_seqlen_q %d > 4: use attn_prefill_paged for longer queries", max_seqlen_q);
  REQUIRE(kv_dtype == ATTN_DTYPE_BF16 || kv_dtype == ATTN_DTYPE_FP8_E4M3FN, ATTN_ERR_UNSUPPORTED,
          "kv_dtype %d not supported (bf16 or fp8 e4m3fn)", kv_dtype);
  const bool fp8 = kv_dtype == ATTN_DTYPE_FP8_E4M3FN;
  REQUIRE(!fp8 || (k_scale != nullptr && v_scale != nullptr), ATTN_ERR_UNSUPPORTED,
          "fp8 KV cache needs per-token k_scale and v_scale");
  REQUIRE(per_tensor_scales == 0 || per_tensor_scales == 1, ATTN_ERR_INVALID,
          "per_tensor_scales must be 0 or 1");
  REQUIRE(!per_tensor_scales || fp8, ATTN_ERR_UNSUPPORTED, "per-tensor scales need an fp8 KV cache");
  REQUIRE(fp8 || (k_scale == nullptr && v_scale == nullptr), ATTN_ERR_UNSUPPORTED,
          "scales are only read with an fp8 KV cache");
  REQUIRE(head_dim == 64 || head_dim == 128, ATTN_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)",
          head_dim);
  REQUIRE(block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128,
          ATTN_ERR_UNSUPPORTED, "block_size %d not supported (16, 32, 64, 128)", block_size);
  REQUIRE(num_q_heads >= 1 && num_kv_heads >= 1, ATTN_ERR_INVALID, "head counts must be positive");
  REQUIRE(num_q_heads % num_kv_heads == 0, ATTN_ERR_INVALID,
          "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", num_q_heads, num_kv_heads);
  REQUIRE(prefill || max_seqlen_q * (num_q_heads / num_kv_heads) <= 64, ATTN_ERR_UNSUPPORTED,
          "max_seqlen_q * (Hq/Hkv) = %d exceeds 64 query rows per KV head",
          max_seqlen_q * (num_q_heads / num_kv_heads));
  REQUIRE(std::isfinite(softmax_scale), ATTN_ERR_INVALID, "softmax_scale is not finite");
  REQUIRE(kv_split_len >= 0, ATTN_ERR_INVALID, "kv_split_len %d is negative", kv_split_len);
  if (kv_split_len > 0) {
    const int unit = block_size > 32 ? block_size : 32;
    REQUIRE(kv_split_len % unit == 0, ATTN_ERR_INVALID,
            "kv_split_len %d must be a multiple of %d", kv_split_len, unit);
    REQUIRE(prefill || kv_split_len <= attn::kDecodeMaxSplit, ATTN_ERR_UNSUPPORTED,
            "kv_split_len %d exceeds %d", kv_split_len, attn::kDecodeMaxSplit);
  }
  if (num_requests == 0) return ok();
  REQUIRE(max_seq_len >= 1, ATTN_ERR_INVALID, "max_seq_len %d must be >= 1", max_seq_len);
  REQUIRE(max_seq_len <= (1 << 30), ATTN_ERR_UNSUPPORTED, "max_seq_len %d exceeds 2^30 tokens", max_seq_len);
  REQUIRE(num_blocks >= 1, ATTN_ERR_INVALID, "num_blocks %d must be >= 1", num_blocks);
  REQUIRE((long)max_pages * block_size >= max_seq_len, ATTN_ERR_INVALID,
          "max_pages %d * block_size %d cannot hold max_seq_len %d", max_pages, block_size, max_seq_len);
  REQ_PTR(q, 16);
  REQ_PTR(cu_seqlens_q, 4);
  REQ_PTR(k_cache, 16);
  REQ_PTR(v_cache, 16);
  if (fp8 && !per_tensor_scales) {
    REQ_PTR(k_scale, 16);
    REQ_PTR(v_scale, 16);
    REQUIRE((long)num_blocks * num_kv_heads * block_size * 4 <= 0xffffffffL, ATTN_ERR_UNSUPPORTED,
            "per-token scale arrays larger than 4 GiB are not supported");
  }
  if (fp8 && per_tensor_scales) { REQ_PTR(k_scale, 4); REQ_PTR(v_scale, 4); }
  if (sink) REQ_PTR(sink, 4);
  if (g_cache) {
    REQ_PTR(g_cache, 16);
    REQUIRE(num_q_heads / num_kv_heads <= 64, ATTN_ERR_UNSUPPORTED,
            "the gate cache is supported with at most 64 query heads per KV head");
    REQUIRE((long)num_blocks * num_q_heads * block_size * 4 <= 0xffffffffL, ATTN_ERR_UNSUPPORTED,
            "gate cache larger than 4 GiB is not supported");
  }
  REQ_PTR(block_table, 4);
  REQ_PTR(seq_lens, 4);
  REQ_PTR(out, 16);
  if (lse) REQ_PTR(lse, 4);
  DecLayout lay = dec_layout(num_requests, max_seqlen_q, max_seq_len, num_q_heads, num_kv_heads,
                             head_dim, block_size, kv_split_len, prefill);
  REQUIRE(lay.total != SIZE_MAX, ATTN_ERR_UNSUPPORTED, "partials of this call would pass 2^60 bytes");
  if (noalloc) {
    // allocation-free path: size the partials for the grid that will run
    // (the balanced split's exact piece count needs the occupancy of its
    // kernel), check them against the scratch before any other runtime
    // call, then use the scratch array
    const bool will_balance = !prefill && kv_split_len == 0 && lay.num_splits > 1 &&
                              (long)num_requests * num_kv_heads * max_seq_len < 0x7fffffffL;
    if (will_balance) {
      attn::DecodeParams q0{};
      q0.Hkv = num_kv_heads;
      q0.row_blocks = (max_seqlen_q * (num_q_heads / num_kv_heads) + 15) / 16;
      q0.g_cache = g_cache;
      const int groups = attn::decode_balanced_groups(q0, head_dim, kv_dtype == ATTN_DTYPE_FP8_E4M3FN);
      if (groups <= 0) return fail(ATTN_ERR_HIP, "occupancy query failed");
      lay = dec_layout(num_requests, max_seqlen_q, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                       block_size, kv_split_len, prefill, groups);
    }
    REQUIRE(lay.total <= (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES, ATTN_ERR_UNSUPPORTED,
            "this call needs %zu bytes of partials, more than the %zu-byte scratch of the "
            "allocation-free decode; use attn_decode_paged with a workspace",
            lay.total, (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES);
    if (lay.total > 0) {
      int st = ATTN_OK;
      workspace = scratch_on_current_device(&st);
      if (workspace == nullptr) return st;
    }
  } else {
    REQUIRE(workspace_bytes >= lay.total, ATTN_ERR_INVALID, "workspace too small: %zu < %zu bytes",
            workspace_bytes, lay.total);
    if (lay.total > 0) REQ_PTR(workspace, 256);
  }
  REQUIRE((long)num_requests * num_kv_heads * lay.num_splits *
                  query_blocks(max_seqlen_q, num_q_heads, num_kv_heads) <= 0x7fffffffL,
          ATTN_ERR_UNSUPPORTED, "more than 2^31 - 1 work items (requests x KV heads x segments x query blocks)");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  attn::DecodeParams p{};
  p.q = q; p.cu_q = cu_seqlens_q; p.k_cache = k_cache; p.v_cache = v_cache;
  p.k_scale = k_scale; p.v_scale = v_scale; p.block_table = block_table; p.seq_lens = seq_lens;
  p.acc = reinterpret_cast<float*>(ws + lay.acc);
  p.m = reinterpret_cast<float*>(ws + lay.m);
  p.l = reinterpret_cast<float*>(ws + lay.l);
  p.R = num_requests; p.max_pages = max_pages; p.Hq = num_q_heads; p.Hkv = num_kv_heads;
  p.B = block_size; p.B_shift = __builtin_ctz((unsigned)block_size); p.split_len = lay.split_len; p.num_splits = lay.num_splits;
  p.scale_log2 = softmax_scale * attn::kLog2e;
  p.row_blocks = (max_seqlen_q * (num_q_heads / num_kv_heads) + 15) / 16;
  p.sink = sink; p.g_cache = g_cache; p.window = window > 0 ? window : 0;
  p.per_tensor = per_tensor_scales;
  if (lay.num_splits == 1) { p.out = out; p.lse = lse; }
  // decode with the library's split: equal shares of all visible keys
  // per workgroup (request lengths vary; fixed-length segments leave the
  // longest ones alone at the end)
  p.balanced = !prefill && kv_split_len == 0 && lay.num_splits > 1 &&
               (long)num_requests * num_kv_heads * max_seq_len < 0x7fffffffL;   // line fits 31 bits
  p.rpu = max_seqlen_q * (num_q_heads / num_kv_heads);
  p.unit_info = reinterpret_cast<int32_t*>(ws + lay.units);
  hipError_t e = prefill && attn::paged_pipe_supported(p, head_dim, fp8, softmax_scale)
                    ? attn::launch_paged_pipe(p, head_dim, fp8, max_seqlen_q, s)
                    : attn::launch_decode_splitk(p, head_dim, fp8, s);
  if (e != hipSuccess) return hip_fail(e, prefill ? "paged prefill launch" : "decode launch");
  if (lay.num_splits == 1) return ok();

  attn::ReduceParams r{};
  r.acc = p.acc; r.m = p.m; r.l = p.l; r.out = out; r.lse = lse;
  r.rows = (long)num_requests * max_seqlen_q * num_q_heads;
  r.num_splits = lay.num_splits; r.dv = head_dim; r.out_fp32 = 0;
  r.seq_lens = seq_lens; r.cu_seqlens_q = cu_seqlens_q; r.num_requests = num_requests;
  r.heads = num_q_heads; r.split_len = lay.split_len;
  r.balanced = p.balanced; r.rpu = p.rpu; r.Hkv = num_kv_heads; r.unit_info = p.unit_info;
  // balanced: a unit's pieces are about its share of the workgroups, plus
  // the pieces cut at its two ends
  r.splits_hint = p.balanced ? p.sk_G / (num_kv_heads * num_requests) + 2 : lay.num_splits;
  e = attn::launch_splitk_reduce(r, s);
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  return ok();
}
}  // namespace

int attn_decode_paged_ext(const void* q, const int32_t* cu_seqlens_q, int num_requests, int max_seqlen_q,
                          const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                          const float* v_scale, int per_tensor_scales, const int32_t* block_table,
                          int max_pages, const int32_t* seq_lens, int max_seq_len, int num_blocks,
                          int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                          float softmax_scale, const float* sink, int window, const float* g_cache,
                          int kv_split_len, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return paged_attention(false, q, cu_seqlens_q, num_requests, max_seqlen_q, k_cache, v_cache, kv_dtype,
                         k_scale, v_scale, per_tensor_scales, block_table, max_pages, seq_lens,
                         max_seq_len, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                         softmax_scale, sink, window, g_cache, kv_split_len, out, lse, workspace,
                         workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free decode: the partials live in this file-scope array (one
// copy per GPU, held until the process ends).  Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, or nullptr (error
// recorded) on a runtime failure.
void* scratch_on_current_device(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { *status = hip_fail(e, "hipGetDevice"); return nullptr; }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(ATTN_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) {
    *status = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}
}  // namespace

int attn_decode_paged_noalloc(const void* q, const int32_t* cu_seqlens_q, int num_requests, int max_seqlen_q,
                              const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                              const float* v_scale, const int32_t* block_table, int max_pages,
                              const int32_t* seq_lens, int max_seq_len, int num_blocks, int block_size,
                              int num_q_heads, int num_kv_heads, int head_dim, float softmax_scale,
                              int kv_split_len, void* out, float* lse, void* stream) {
  return paged_attention(false, q, cu_seqlens_q, num_requests, max_seqlen_q, k_cache, v_cache, kv_dtype,
                         k_scale, v_scale, 0, block_table, max_pages, seq_lens, max_seq_len, num_blocks,
                         block_size, num_q_heads, num_kv_heads, head_dim, softmax_scale, nullptr, 0, nullptr,
                         kv_split_len, out, lse, nullptr, 0, stream, true);
}

size_t attn_prefill_paged_workspace_size(int num_requests, int max_seqlen_q, int max_seq_len,
                                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                         int kv_split_len) {
  if (num_requests <= 0 || max_seqlen_q <= 0 || max_seq_len <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || kv_split_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  return dec_layout(num_requests, max_seqlen_q, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                    block_size, kv_split_len, true).total;
}

int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q, int num_requests, int max_seqlen_q,
                       const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                       const float* v_scale, int per_tensor_scales, const int32_t* block_table,
                       int max_pages, const int32_t* seq_lens, int max_seq_len, int num_blocks,
                       int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                       float softmax_scale, const float* sink, int window, const float* g_cache,
                       int kv_split_len, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return paged_attention(true, q, cu_seqlens_q, num_requests, max_seqlen_q, k_cache, v_cache, kv_dtype,
                         k_scale, v_scale, per_tensor_scales, block_table, max_pages, seq_lens,
                         max_seq_len, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                         softmax_scale, sink, window, g_cache, kv_split_len, out, lse, workspace,
                         workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
int attn_splitk_reduce(const float* acc, const float* m, const float* l, int rows, int num_splits,
                       int head_dim_v, void* out, int out_dtype, float* lse, void* stream) {
  REQUIRE(rows >= 0, ATTN_ERR_INVALID, "rows %d is negative", rows);
  REQUIRE(num_splits >= 1, ATTN_ERR_INVALID, "num_splits %d must be >= 1", num_splits);
  REQUIRE(head_dim_v == 64 || head_dim_v == 128 || head_dim_v == 256 || head_dim_v == 512,
          ATTN_ERR_UNSUPPORTED, "head_dim_v %d not supported (64, 128, 256, 512)", head_dim_v);
  REQUIRE(out_dtype == ATTN_DTYPE_BF16 || out_dtype == ATTN_DTYPE_FP32, ATTN_ERR_UNSUPPORTED,
          "out_dtype %d not supported (bf16 or fp32)", out_dtype);
  if (rows == 0) return ok();
  REQ_PTR(acc, 16);
  REQ_PTR(m, 4);
  REQ_PTR(l, 4);
  REQ_PTR(out, 16);
  if (lse) REQ_PTR(lse, 4);
  attn::ReduceParams r{};
  r.acc = acc; r.m = m; r.l = l; r.out = out; r.lse = lse; r.rows = rows;
  r.num_splits = num_splits; r.dv = head_dim_v; r.out_fp32 = out_dtype == ATTN_DTYPE_FP32;
  hipError_t e = attn::launch_splitk_reduce(r, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  return ok();
}

int attn_kv_cache_write_fp8(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                            int num_tokens, int num_kv_heads, int head_dim, void* k_cache,
                            void* v_cache, float* k_scale, float* v_scale, int num_blocks,
                            int block_size, void* stream) {
  REQUIRE(num_tokens >= 0 && num_blocks >= 0, ATTN_ERR_INVALID,
          "negative size (num_tokens=%d num_blocks=%d)", num_tokens, num_blocks);
  REQUIRE(num_kv_heads >= 1, ATTN_ERR_INVALID, "num_kv_heads %d must be positive", num_kv_heads);
  REQUIRE(head_dim == 64 || head_dim == 128, ATTN_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)",
          head_dim);
  REQUIRE(block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128,
          ATTN_ERR_UNSUPPORTED, "block_size %d not supported (16, 32, 64, 128)", block_size);
  REQUIRE((long)num_blocks * block_size <= 0x7fffffffL, ATTN_ERR_UNSUPPORTED,
          "num_blocks * block_size exceeds the int32 slot range");
  if (num_tokens == 0) return ok();
  REQ_PTR(k_new, 16);
  REQ_PTR(v_new, 16);
  REQ_PTR(slot_mapping, 4);
  REQ_PTR(k_cache, 8);
  REQ_PTR(v_cache, 8);
  REQ_PTR(k_scale, 4);
  REQ_PTR(v_scale, 4);
  attn::KvWriteParams p{};
  p.k_new = k_new; p.v_new = v_new; p.slot_mapping = slot_mapping;
  p.k_cache = k_cache; p.v_cache = v_cache; p.k_scale = k_scale; p.v_scale = v_scale;
  p.N = num_tokens; p.Hkv = num_kv_heads; p.NB = num_blocks; p.B = block_size;
  hipError_t e = attn::launch_kv_cache_write_fp8(p, head_dim, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv cache write launch");
  return ok();
}

}  // extern "C"
