"""Causal softmax attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libattn.so`` (C ABI in include/attn.h).  The
Python side only marshals arguments: it checks torch dtypes, devices and
contiguity (which the C side cannot see), allocates outputs and the
workspace with torch, and passes raw device pointers plus the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback path.  If the library is missing, importing this package
raises at once.

Entry points (same names as the C functions):
  attn_fwd_varlen    packed variable-length causal attention forward
  attn_bwd_varlen    its gradients dq, dk, dv, dsink, dg
  attn_decode_paged  paged decode of 1..4 query tokens per request
  attn_splitk_reduce log-sum-exp merge of split-K partials
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["attn_fwd_varlen", "attn_bwd_varlen", "attn_decode_paged", "attn_decode_paged_noalloc",
           "attn_prefill_paged",
           "attn_splitk_reduce", "attn_kv_cache_write_fp8", "attn_fwd_workspace_size",
           "attn_bwd_workspace_size", "attn_decode_workspace_size",
           "attn_prefill_paged_workspace_size",
           "ATTN_DTYPE_BF16", "ATTN_DTYPE_FP8_E4M3FN", "ATTN_DTYPE_FP32",
           "ATTN_BWD_DETERMINISTIC", "ATTN_BWD_FUSED_DQ", "ATTN_BWD_RECOMPUTE_DQ",
           "AttnError", "lib_path", "library"]

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, -1, -2, -3
ATTN_DTYPE_BF16, ATTN_DTYPE_FP8_E4M3FN, ATTN_DTYPE_FP32 = 0, 1, 2
ATTN_BWD_DETERMINISTIC, ATTN_BWD_FUSED_DQ, ATTN_BWD_RECOMPUTE_DQ = 1, 2, 4

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree library this package loads."""
    return os.path.join(_HERE, "libattn.so")


class AttnError(RuntimeError):
    """A HIP runtime failure reported by the library."""


_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "attn_status_string": ([_c_int], ctypes.c_char_p),
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_version": ([], ctypes.c_char_p),
    "attn_fwd_workspace_size": ([_c_int, _c_int, _c_int], _c_size),
    "attn_fwd_varlen": ([_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                         _c_int, _c_float, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp], _c_int),
    "attn_bwd_workspace_size": ([_c_int] * 10, _c_size),
    "attn_bwd_varlen": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                         _c_int, _c_int, _c_int, _c_float, _c_int, _vp, _vp, _vp, _vp, _vp,
                         _vp, _vp, _c_int, _vp, _c_size, _vp], _c_int),
    "attn_decode_workspace_size": ([_c_int] * 8, _c_size),
    "attn_decode_paged": ([_vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int,
                           _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                           _c_int, _vp, _vp, _vp, _c_size, _vp], _c_int),
    "attn_decode_paged_ext": ([_vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _c_int,
                               _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _vp,
                               _c_int, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp], _c_int),
    "attn_decode_paged_noalloc": ([_vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _c_int,
                                   _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                   _c_int, _vp, _vp, _vp], _c_int),
    "attn_prefill_paged_workspace_size": ([_c_int] * 8, _c_size),
    "attn_prefill_paged": ([_vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _c_int,
                            _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _vp,
                            _c_int, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp], _c_int),
    "attn_splitk_reduce": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp], _c_int),
    "attn_kv_cache_write_fp8": ([_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_int,
                                 _c_int, _vp], _c_int),
}


def _load():
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python causal_softmax_attention_amd/build.py` "
            "(hipcc for gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


library = _load()


def _check(status: int, name: str):
    if status == ATTN_OK:
        return
    detail = library.attn_last_error().decode()
    msg = f"{name}: {library.attn_status_string(status).decode()}: {detail}"
    if status == ATTN_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status == ATTN_ERR_INVALID:
        raise ValueError(msg)
    raise AttnError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device=None, ndim=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strided tensors are not supported)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def attn_fwd_workspace_size(total_tokens, num_q_heads, has_gate) -> int:
    return int(library.attn_fwd_workspace_size(total_tokens, num_q_heads, int(bool(has_gate))))


def attn_bwd_workspace_size(total_tokens, num_seqs, max_seqlen, num_q_heads, head_dim_qk, head_dim_v,
                            window, has_gate, has_sink, flags=0) -> int:
    return int(library.attn_bwd_workspace_size(total_tokens, num_seqs, max_seqlen, num_q_heads,
                                               head_dim_qk, head_dim_v, window, int(bool(has_gate)),
                                               int(bool(has_sink)), int(flags)))


def attn_decode_workspace_size(num_requests, max_seqlen_q, max_seq_len, num_q_heads,
                               num_kv_heads, head_dim, block_size, kv_split_len=0) -> int:
    return int(library.attn_decode_workspace_size(num_requests, max_seqlen_q, max_seq_len,
                                                  num_q_heads, num_kv_heads, head_dim,
                                                  block_size, kv_split_len))


def attn_prefill_paged_workspace_size(num_requests, max_seqlen_q, max_seq_len, num_q_heads,
                                      num_kv_heads, head_dim, block_size, kv_split_len=0) -> int:
    return int(library.attn_prefill_paged_workspace_size(num_requests, max_seqlen_q, max_seq_len,
                                                         num_q_heads, num_kv_heads, head_dim,
                                                         block_size, kv_split_len))


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, window=0,
                    sink=None, g=None, out=None, lse=None):
    """Forward over packed sequences.  q [T, Hq, d_qk], k [T, Hkv, d_qk],
    v [T, Hkv, d_v] bf16; cu_seqlens int32 [N+1]; sink fp32 [Hq] or None;
    g fp32 [T, Hq] log gates or None; window <= 0 for none.  Returns
    (o bf16 [T, Hq, d_v], lse fp32 [T, Hq])."""
    dev = q.device
    _need(q, "q", torch.bfloat16, None, 3)
    _need(k, "k", torch.bfloat16, dev, 3)
    _need(v, "v", torch.bfloat16, dev, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
    T, Hq, dqk = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    if k.shape != (T, Hkv, dqk) or v.shape[:2] != (T, Hkv):
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev, 1)
    if g is not None:
        _need(g, "g", torch.float32, dev, 2)
        if tuple(g.shape) != (T, Hq):
            raise ValueError(f"g must be [{T}, {Hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    if out is None:
        out = torch.empty((T, Hq, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    ws_n = attn_fwd_workspace_size(T, Hq, g is not None)
    ws = _workspace(ws_n, dev)
    st = library.attn_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen),
        T, Hq, Hkv, dqk, dv, float(softmax_scale), int(window), _ptr(sink), _ptr(g),
        _ptr(out), _ptr(lse), _ptr(ws), ws_n, _stream(dev))
    _check(st, "attn_fwd_varlen")
    return out, lse


def attn_bwd_varlen(q, k, v, o, do, lse, cu_seqlens, max_seqlen, softmax_scale=None,
                    window=0, sink=None, g=None, flags=0):
    """Gradients of attn_fwd_varlen given dO.  flags: 0 / ATTN_BWD_DETERMINISTIC
    (two-pass, no atomics; for d_v 512, and d_qk 256 with d_v 128 / 256, dS
    is stored between the passes unless ATTN_BWD_RECOMPUTE_DQ is added) or ATTN_BWD_FUSED_DQ (dQ fused into the
    dK/dV pass with fp32 atomics, d_qk <= 128).  Returns (dq, dk, dv bf16, dsink fp32
    [Hq] or None, dg fp32 [T, Hq] or None)."""
    dev = q.device
    _need(q, "q", torch.bfloat16, None, 3)
    _need(k, "k", torch.bfloat16, dev, 3)
    _need(v, "v", torch.bfloat16, dev, 3)
    _need(o, "o", torch.bfloat16, dev, 3)
    _need(do, "do", torch.bfloat16, dev, 3)
    _need(lse, "lse", torch.float32, dev, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
    T, Hq, dqk = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    if o.shape != (T, Hq, dv) or do.shape != (T, Hq, dv) or lse.shape != (T, Hq):
        raise ValueError("o, do must be [T, Hq, d_v] and lse [T, Hq]")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev, 1)
    if g is not None:
        _need(g, "g", torch.float32, dev, 2)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dsink = torch.empty((Hq,), dtype=torch.float32, device=dev) if sink is not None else None
    dg = torch.empty((T, Hq), dtype=torch.float32, device=dev) if g is not None else None
    ws_n = attn_bwd_workspace_size(T, cu_seqlens.numel() - 1, int(max_seqlen), Hq, dqk, dv, int(window),
                                   g is not None, sink is not None, flags)
    ws = _workspace(ws_n, dev)
    st = library.attn_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, int(max_seqlen), T, Hq, Hkv, dqk, dv, float(softmax_scale),
        int(window), _ptr(sink), _ptr(g), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(dsink), _ptr(dg),
        int(flags), _ptr(ws), ws_n, _stream(dev))
    _check(st, "attn_bwd_varlen")
    return dq, dk, dvv, dsink, dg


def _paged(prefill, q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype, k_scale, v_scale,
           block_table, seq_lens, max_seq_len, softmax_scale, kv_split_len, return_lse, out,
           sink, window, g_cache):
    dev = q.device
    _need(q, "q", torch.bfloat16, None, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    if kv_dtype == ATTN_DTYPE_FP8_E4M3FN:
        cache_dtypes = (torch.uint8, torch.float8_e4m3fn)
    else:
        cache_dtypes = (torch.bfloat16,)
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype not in cache_dtypes:
            raise ValueError(f"{name} dtype {c.dtype} does not match kv_dtype {kv_dtype}")
        _need(c, name, c.dtype, dev, 4)
    for name, s in (("k_scale", k_scale), ("v_scale", v_scale)):
        if s is not None:
            _need(s, name, torch.float32, dev, None)   # [NB, Hkv, B], or [1] per tensor
    Tq, Hq, D = q.shape
    NB, Hkv, B, Dc = k_cache.shape
    if v_cache.shape != k_cache.shape or Dc != D:
        raise ValueError("k_cache and v_cache must both be [NB, Hkv, B, D] with q's D")
    per_tensor = k_scale is not None and k_scale.numel() == 1
    for s in (k_scale, v_scale):
        if s is None:
            continue
        if per_tensor:
            if s.numel() != 1:
                raise ValueError("per-tensor scales: both k_scale and v_scale must hold one value")
        elif tuple(s.shape) != (NB, Hkv, B):
            raise ValueError(f"scales must be [{NB}, {Hkv}, {B}] (or one value each)")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev, 1)
    if g_cache is not None:
        _need(g_cache, "g_cache", torch.float32, dev, 3)
        if tuple(g_cache.shape) != (NB, Hq, B):
            raise ValueError(f"g_cache must be [{NB}, {Hq}, {B}]")
    R = seq_lens.numel()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev) if return_lse else None
    ws_fn = attn_prefill_paged_workspace_size if prefill else attn_decode_workspace_size
    ws_n = ws_fn(R, int(max_seqlen_q), int(max_seq_len), Hq, Hkv, D, B, int(kv_split_len))
    ws = _workspace(ws_n, dev)
    entry = library.attn_prefill_paged if prefill else library.attn_decode_paged_ext
    st = entry(
        _ptr(q), _ptr(cu_seqlens_q), R, int(max_seqlen_q), _ptr(k_cache), _ptr(v_cache),
        int(kv_dtype), _ptr(k_scale), _ptr(v_scale), int(per_tensor), _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), int(max_seq_len), NB, B, Hq, Hkv, D,
        float(softmax_scale), _ptr(sink), int(window), _ptr(g_cache), int(kv_split_len),
        _ptr(out), _ptr(lse), _ptr(ws), ws_n, _stream(dev))
    _check(st, "attn_prefill_paged" if prefill else "attn_decode_paged")
    return (out, lse) if return_lse else out


def attn_decode_paged(q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype,
                      k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      softmax_scale=None, kv_split_len=0, return_lse=False, out=None,
                      sink=None, window=0, g_cache=None):
    """Paged decode.  q bf16 [Tq, Hq, D]; k_cache / v_cache [NB, Hkv, B, D]
    as bf16 or as uint8 / float8_e4m3fn codes; k_scale / v_scale fp32
    [NB, Hkv, B] for fp8 (None for bf16); block_table int32 [R, max_pages];
    seq_lens int32 [R].  Returns out bf16 [Tq, Hq, D] (and lse fp32 [Tq, Hq]).
    Optional: one-element k_scale / v_scale = per-tensor fp8 scales; sink fp32
    [Hq]; window (> 0); g_cache fp32 [NB, Hq, B] cumulative log gates."""
    return _paged(False, q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                  block_table, seq_lens, max_seq_len, softmax_scale, kv_split_len, return_lse, out,
                  sink, window, g_cache)


def attn_decode_paged_noalloc(q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype,
                              k_scale, v_scale, block_table, seq_lens, max_seq_len, out, lse=None,
                              softmax_scale=None, kv_split_len=0):
    """attn_decode_paged without a workspace: the split-K partials live in the
    library's own per-GPU scratch, so neither this call nor the library
    allocates anything.  The caller passes the outputs: out bf16 [Tq, Hq, D]
    and optionally lse fp32 [Tq, Hq].  Calls that may overlap on one GPU
    share that scratch and must be serialised.  Returns out."""
    dev = q.device
    _need(q, "q", torch.bfloat16, None, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    Tq, Hq, D = q.shape
    NB, Hkv, B, Dc = k_cache.shape
    if v_cache.shape != k_cache.shape or Dc != D:
        raise ValueError("k_cache and v_cache must both be [NB, Hkv, B, D] with q's D")
    _need(out, "out", torch.bfloat16, dev, 3)
    if tuple(out.shape) != (Tq, Hq, D):
        raise ValueError(f"out must be [{Tq}, {Hq}, {D}]")
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    st = library.attn_decode_paged_noalloc(
        _ptr(q), _ptr(cu_seqlens_q), seq_lens.numel(), int(max_seqlen_q), _ptr(k_cache), _ptr(v_cache),
        int(kv_dtype), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), int(max_seq_len), NB, B, Hq, Hkv, D, float(softmax_scale), int(kv_split_len),
        _ptr(out), _ptr(lse), _stream(dev))
    _check(st, "attn_decode_paged_noalloc")
    return out


def attn_prefill_paged(q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype,
                       k_scale, v_scale, block_table, seq_lens, max_seq_len,
                       softmax_scale=None, kv_split_len=0, return_lse=False, out=None,
                       sink=None, window=0, g_cache=None):
    """Paged prefill: as attn_decode_paged with any number of new tokens per
    request (each request's new tokens already in its cache)."""
    return _paged(True, q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                  block_table, seq_lens, max_seq_len, softmax_scale, kv_split_len, return_lse, out,
                  sink, window, g_cache)


def attn_splitk_reduce(acc, m, l, out_dtype=torch.float32, return_lse=True):
    """Merge partials acc fp32 [rows, S, Dv], m / l fp32 [rows, S].  Returns
    (out [rows, Dv] of out_dtype, lse fp32 [rows] or None)."""
    dev = acc.device
    _need(acc, "acc", torch.float32, None, 3)
    _need(m, "m", torch.float32, dev, 2)
    _need(l, "l", torch.float32, dev, 2)
    rows, S, Dv = acc.shape
    if tuple(m.shape) != (rows, S) or tuple(l.shape) != (rows, S):
        raise ValueError("m and l must be [rows, num_splits]")
    code = {torch.float32: ATTN_DTYPE_FP32, torch.bfloat16: ATTN_DTYPE_BF16}.get(out_dtype)
    if code is None:
        raise NotImplementedError(f"out_dtype {out_dtype} not supported")
    out = torch.empty((rows, Dv), dtype=out_dtype, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev) if return_lse else None
    st = library.attn_splitk_reduce(_ptr(acc), _ptr(m), _ptr(l), rows, S, Dv, _ptr(out), code,
                                    _ptr(lse), _stream(dev))
    _check(st, "attn_splitk_reduce")
    return out, lse


def attn_kv_cache_write_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Quantise new tokens into the paged fp8 cache in place.  k_new / v_new
    bf16 [N, Hkv, D]; slot_mapping int32 [N] (page * block_size + offset,
    negative = skip); k_cache / v_cache uint8 or float8_e4m3fn [NB, Hkv, B, D];
    k_scale / v_scale fp32 [NB, Hkv, B]."""
    dev = k_new.device
    _need(k_new, "k_new", torch.bfloat16, None, 3)
    _need(v_new, "v_new", torch.bfloat16, dev, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, dev, 1)
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must hold fp8 bytes (uint8 or float8_e4m3fn), got {c.dtype}")
        _need(c, name, c.dtype, dev, 4)
    _need(k_scale, "k_scale", torch.float32, dev, 3)
    _need(v_scale, "v_scale", torch.float32, dev, 3)
    N, Hkv, D = k_new.shape
    if tuple(v_new.shape) != (N, Hkv, D) or slot_mapping.numel() != N:
        raise ValueError("k_new, v_new must be [N, Hkv, D] and slot_mapping [N]")
    NB, Hc, B, Dc = k_cache.shape
    if (Hc, Dc) != (Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [NB, Hkv, B, D] with the new tokens' Hkv and D")
    for s_ in (k_scale, v_scale):
        if tuple(s_.shape) != (NB, Hkv, B):
            raise ValueError(f"scales must be [{NB}, {Hkv}, {B}]")
    st = library.attn_kv_cache_write_fp8(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), N, Hkv, D,
                                         _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                         NB, B, _stream(dev))
    _check(st, "attn_kv_cache_write_fp8")
