// Per-token fp8 KV-cache write.
//
// Method (ROCm/aiter PR #6660, commit messages and "Technical details"): the
// paged KV cache holds fp8 e4m3fn codes with one fp32 scale per token and KV
// head, and decode multiplies codes by those scales.  For each new token and
// KV head, separately for K and V: amax = max |x|, scale = amax / 448 (1 for
// an all-zero row), code = round-to-nearest-even e4m3fn of x / scale
// (clamped to +-448), written to the token's slot of the cache and scales.
//
// gfx950 mapping: D/8 lanes per (token, head) row, 16 bytes of K and of V
// per lane; the row maximum is a butterfly over those lanes; two codes per
// v_cvt_pk_fp8_f32.  HBM-bound: 2 x (2D read + D written + 4) bytes per row.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int D>
__global__ __launch_bounds__(256) void kv_cache_write_fp8_kernel(KvWriteParams p) {
  constexpr int LPR = D / 8;                 // lanes per (token, head) row
  constexpr int RPB = 256 / LPR;             // rows per workgroup
  const int t = threadIdx.x, sub = t % LPR;
  const long row = (long)blockIdx.x * RPB + t / LPR;   // token * Hkv + head
  if (row >= (long)p.N * p.Hkv) return;
  const int tok = (int)(row / p.Hkv), h = (int)(row % p.Hkv);
  const int slot = p.slot_mapping[tok];
  if (slot < 0 || slot >= p.NB * p.B) return;        // padding token / out of range: skipped
  const int page = slot / p.B, off = slot % p.B;
  const long dst = ((long)page * p.Hkv + h) * p.B + off;   // (page, head, slot) index
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const bf16* src = reinterpret_cast<const bf16*>(which ? p.v_new : p.k_new) + row * D + 8 * sub;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(src);
    float f[8], amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = (float)x[e];
      amax = fmaxf(amax, fabsf(f[e]));
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    int w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(f[4 * k + e] / scale, -448.0f), 448.0f);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
      w[k] = word;
    }
    uint8_t* cache = reinterpret_cast<uint8_t*>(which ? p.v_cache : p.k_cache);
    *reinterpret_cast<i32x2*>(cache + dst * D + 8 * sub) = i32x2{w[0], w[1]};
    if (sub == 0) (which ? p.v_scale : p.k_scale)[dst] = scale;
  }
}

hipError_t launch_kv_cache_write_fp8(const KvWriteParams& p, int head_dim, hipStream_t st) {
  const long rows = (long)p.N * p.Hkv;
  if (rows == 0) return hipSuccess;
  if (head_dim == 128) {
    kv_cache_write_fp8_kernel<128><<<dim3((unsigned)((rows + 15) / 16)), 256, 0, st>>>(p);
  } else if (head_dim == 64) {
    kv_cache_write_fp8_kernel<64><<<dim3((unsigned)((rows + 31) / 32)), 256, 0, st>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
