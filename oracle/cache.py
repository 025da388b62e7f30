"""CPU oracle for the per-token fp8 KV-cache write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark may
call it.  It shares no code with the HIP library.

What it computes (ROCm/aiter PR #6660, commit messages and "Technical
details": the KV cache holds fp8 codes with one scale per token and KV head,
and decode multiplies the codes by those scales): for each new token t and KV
head h, separately for K and for V,

    amax  = max_d |x[t, h, d]|
    scale = amax / 448           (448 = largest finite e4m3fn value;
                                  scale = 1 when amax = 0)
    code  = e4m3fn(x / scale)    (round to nearest even)

written to slot slot_mapping[t] (page = slot // B, offset = slot % B) of the
[num_blocks, Hkv, B, D] cache and of the [num_blocks, Hkv, B] scales.
Negative slots (padding tokens) are skipped.

Readings (the pages give the scale layout but not the quantiser): the scale
is amax / 448 per (token, KV head); the code is the round-to-nearest-even
e4m3fn value of x / scale.  Because a floating-point computation decides an
integer here, every step is taken in float32 exactly as the kernel takes it
(amax, the division by 448, the division x / scale), and the quotient is
clamped to +-448 before encoding.
"""
from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0


def e4m3fn_encode(v) -> np.ndarray:
    """Round-to-nearest-even OCP e4m3fn codes of float values with
    |v| <= 448 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
    infinities; subnormals below 2^-6 in steps of 2^-9).  NaN maps to 0x7F."""
    x = np.asarray(v, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.uint8)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # subnormal range: multiples of 2^-9 below 2^-6 (an m of 8 is 2^-6 itself)
    sub = a < 2.0 ** -6
    m_sub = np.rint(a / 2.0 ** -9)                      # round half to even
    code_sub = np.where(m_sub >= 8, 1 << 3, m_sub).astype(np.int64)
    # normal range: a = (1 + m/8) 2^e, e in [-6, 8]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a)))
    frac = np.where(sub, 1.0, a) / 2.0 ** e               # in [1, 2)
    m = np.rint((frac - 1.0) * 8.0)                        # round half to even
    e = np.where(m >= 8, e + 1, e)
    m = np.where(m >= 8, 0, m)
    code_norm = ((e + 7).astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(sub, code_sub, code_norm)
    out = (code.astype(np.uint8) | sign)
    out = np.where(nan, np.uint8(0x7F), out)
    return out.astype(np.uint8)


def quantize_token_heads(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row fp8 quantisation of x [..., D] (values exactly representable in
    float32): returns (codes uint8 [..., D], scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3FN_MAX), np.float32(1.0)).astype(np.float32)
    q = (x32 / scale[..., None]).astype(np.float32)
    q = np.clip(q, -np.float32(E4M3FN_MAX), np.float32(E4M3FN_MAX))
    return e4m3fn_encode(q), scale


def cache_write_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Write new tokens into copies of the cache.

    k_new, v_new: [N, Hkv, D] values (bf16 upcast); slot_mapping: [N] int;
    k_cache, v_cache: uint8 [NB, Hkv, B, D]; k_scale, v_scale: float32
    [NB, Hkv, B].  Returns the four updated arrays (inputs are not modified).
    """
    kc, vc = np.array(k_cache, dtype=np.uint8), np.array(v_cache, dtype=np.uint8)
    ks, vs = np.array(k_scale, dtype=np.float32), np.array(v_scale, dtype=np.float32)
    B = kc.shape[2]
    kq, ksc = quantize_token_heads(k_new)
    vq, vsc = quantize_token_heads(v_new)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        page, off = divmod(int(slot), B)
        kc[page, :, off, :] = kq[t]
        vc[page, :, off, :] = vq[t]
        ks[page, :, off] = ksc[t]
        vs[page, :, off] = vsc[t]
    return kc, vc, ks, vs
