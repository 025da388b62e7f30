"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times.  Where the float64 oracle cannot redo everything in seconds
it checks sampled outputs, each computed from the definition on its own:

  1. dense 128 tokens, GQA 4, d 64, sink: everything.
  2. packed varlen, 32/8 heads, d 128, window 1024, sink, gates: the whole
     forward; backward for two KV-head groups (dq, dk, dv, dg of their heads)
     and dsink of their query heads, through the two-pass and the fused-dQ
     paths.
  3. paged single-query decode, 64 requests up to 32K context, fp8 per-token
     scales, page 16: eight sampled requests (all their query rows).
  4. 3 x 4-token verify over ~227K contexts, page 128, bf16 and fp8: all rows.
  5. 4 x 8192 tokens, 16/4 heads, d_qk 256 / d_v 512, sink, gates: forward
     rows sampled from every sequence; backward (dq, dk, dv, dg) for KV head
     1 of sequence 0; dsink of heads 4..7 from the definition
     dsink_h = -sum_i psink_i <dO_i, o_i> with o, lse from the forward oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.util import rel_rms

pytestmark = pytest.mark.gpu
TOL = 5e-3
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def A():
    import causal_softmax_attention_amd as A
    return A


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _run_prefill(A, x):
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window, x.sink, x.g)
    grads = A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale,
                              x.window, x.sink, x.g)
    torch.cuda.synchronize()
    return o, lse, grads


def test_dense_128_full(A):
    _say("[case] dense 128 tokens gqa4 d64 full")
    x = synth.dense_128_gqa4(device=DEV)
    o, lse, (dq, dk, dv, ds, dg) = _run_prefill(A, x)
    ro, rl = oracle.forward(x.q, x.k, x.v, x.cu_seqlens, x.scale, x.window, x.sink, x.g)
    rq, rk, rv, rs, _ = oracle.backward(x.q, x.k, x.v, x.do, x.cu_seqlens, x.scale, x.window, x.sink, x.g)
    errs = dict(o=rel_rms(_np(o), ro), dq=rel_rms(_np(dq), rq), dk=rel_rms(_np(dk), rk),
                dv=rel_rms(_np(dv), rv), dsink=rel_rms(_np(ds), rs))
    _say("   ", errs)
    assert dg is None
    assert max(errs.values()) <= TOL
    assert np.max(np.abs(_np(lse) - rl)) < 1e-3


_CFG2_KVS = [0, 5]
_cfg2_ref_cache = {}


def _cfg2_backward_ref(x):
    # the oracle's backward for two KV-head groups, shared by the two paths
    if "ref" not in _cfg2_ref_cache:
        _cfg2_ref_cache["ref"] = oracle.backward(x.q, x.k, x.v, x.do, x.cu_seqlens, x.scale, x.window,
                                                 x.sink, x.g, kv_heads=_CFG2_KVS)
    return _cfg2_ref_cache["ref"]


def _cfg2_check_backward(x, grads):
    dq, dk, dv, ds, dg = grads
    rq, rk, rv, rs, rg = _cfg2_backward_ref(x)
    kvs = _CFG2_KVS
    heads = [h for kv in kvs for h in range(kv * 4, kv * 4 + 4)]
    errs = dict(dq=rel_rms(_np(dq)[:, heads], rq[:, heads]),
                dk=rel_rms(_np(dk)[:, kvs], rk[:, kvs]),
                dv=rel_rms(_np(dv)[:, kvs], rv[:, kvs]),
                dsink=rel_rms(_np(ds)[heads], rs[heads]),
                dg=rel_rms(_np(dg)[:, heads], rg[:, heads]))
    _say("   ", {k: f"{v:.3e}" for k, v in errs.items()})
    assert max(errs.values()) <= TOL


def test_varlen_8seq_window_full_forward_sampled_backward(A):
    _say("[case] varlen 8 seqs window 1024 sink gate")
    x = synth.varlen_8seq_window1024(device=DEV)
    o, lse, grads = _run_prefill(A, x)
    ro, rl = oracle.forward(x.q, x.k, x.v, x.cu_seqlens, x.scale, x.window, x.sink, x.g)
    e_o = rel_rms(_np(o), ro)
    _say(f"    o={e_o:.3e} lse max abs={np.max(np.abs(_np(lse) - rl)):.2e}")
    assert e_o <= TOL
    assert np.max(np.abs(_np(lse) - rl)) < 1e-3
    _cfg2_check_backward(x, grads)


def test_varlen_8seq_window_fused_dq_sampled_backward(A):
    # the same workload through the fused-dQ backward (fp32 atomics)
    _say("[case] varlen 8 seqs window 1024 sink gate, fused dQ")
    x = synth.varlen_8seq_window1024(device=DEV)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window, x.sink, x.g)
    grads = A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale,
                              x.window, x.sink, x.g, flags=A.ATTN_BWD_FUSED_DQ)
    torch.cuda.synchronize()
    _cfg2_check_backward(x, grads)


def test_decode_64req_sampled_requests(A):
    _say("[case] decode 64 requests fp8 page 16")
    d = synth.decode_64req_fp8(device=DEV)
    out, lse = A.attn_decode_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype,
                                   d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len,
                                   d.scale, return_lse=True)
    torch.cuda.synchronize()
    L = d.seq_lens.cpu().numpy()
    order = np.argsort(L)
    reqs = sorted(set([int(order[0]), int(order[1]), int(order[-1]), int(order[-2])] +
                      [int(i) for i in np.random.default_rng(0).choice(len(L), 4, replace=False)]))
    # the oracle reads only the sampled requests' pages
    kc, vc = d.k_cache.cpu(), d.v_cache.cpu()
    ks, vs = d.k_scale.cpu(), d.v_scale.cpu()
    ro, rl = oracle.decode_paged(d.q, d.cu_seqlens_q, kc, vc, d.block_table, d.seq_lens, d.scale, True,
                                 ks, vs, requests=reqs)
    rows = [int(d.cu_seqlens_q[r]) for r in reqs]
    o = _np(out)[rows]
    err = rel_rms(o, ro[rows])
    bias = float(np.sum(o * ro[rows]) / np.sum(ro[rows] ** 2) - 1)
    _say(f"    requests {reqs} (L {[int(L[r]) for r in reqs]}): rel_rms={err:.3e} bias={bias:.2e}")
    assert err <= TOL and abs(bias) < 1e-3
    assert np.max(np.abs(_np(lse)[rows] - rl[rows])) < 1e-3
    assert torch.isfinite(out).all().item()


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_FP8_E4M3FN], ids=["bf16", "fp8"])
def test_verify_3x4_227k(A, kv):
    _say(f"[case] verify 3x4 tokens 227K context {kv}")
    d = synth.verify_3x4_227k(kv_dtype=kv, device=DEV)
    out, lse = A.attn_decode_paged(d.q, d.cu_seqlens_q, 4, d.k_cache, d.v_cache, kv, d.k_scale, d.v_scale,
                                   d.block_table, d.seq_lens, d.max_seq_len, d.scale, return_lse=True)
    torch.cuda.synchronize()
    fp8 = kv == synth.KV_FP8_E4M3FN
    ro, rl = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache.cpu(), d.v_cache.cpu(), d.block_table,
                                 d.seq_lens, d.scale, fp8,
                                 None if not fp8 else d.k_scale.cpu(), None if not fp8 else d.v_scale.cpu())
    o = _np(out)
    err = rel_rms(o, ro)
    bias = float(np.sum(o * ro) / np.sum(ro * ro) - 1)
    _say(f"    rel_rms={err:.3e} bias={bias:.2e}")
    assert err <= TOL and abs(bias) < 1e-3
    assert np.max(np.abs(_np(lse) - rl)) < 1e-3


def test_varlen_wide_heads_sampled(A):
    _say("[case] varlen 4x8192 d_qk 256 d_v 512")
    x = synth.varlen_4x8192_wide_heads(device=DEV)
    o, lse, (dq, dk, dv, ds, dg) = _run_prefill(A, x)
    cu = x.cu_seqlens.cpu().numpy()
    rng = np.random.default_rng(5)
    toks = sorted(set(int(t) for t in np.concatenate(
        [cu[:-1], cu[1:] - 1, rng.integers(0, int(cu[-1]), 24)])))
    heads = list(range(16))
    ro, rl = oracle.forward_rows(x.q, x.k, x.v, x.cu_seqlens, x.scale, toks, heads, 0, x.sink, x.g)
    e_o = rel_rms(_np(o)[toks][:, heads], ro)
    _say(f"    forward rows {len(toks)} x 16 heads: o={e_o:.3e}")
    assert e_o <= TOL
    assert np.max(np.abs(_np(lse)[toks][:, heads] - rl)) < 1e-3
    # backward of KV head 1 (query heads 4..7) over sequence 0
    a, b = int(cu[0]), int(cu[1])
    c1 = np.array([0, b - a])
    sl = lambda t: t[a:b].cpu()
    rq, rk, rv, _, rg = oracle.backward(sl(x.q), sl(x.k), sl(x.v), sl(x.do), c1, x.scale, 0, x.sink.cpu(),
                                        sl(x.g), kv_heads=[1])
    hs = [4, 5, 6, 7]
    errs = dict(dq=rel_rms(_np(dq)[a:b][:, hs], rq[:, hs]), dk=rel_rms(_np(dk)[a:b][:, 1], rk[:, 1]),
                dv=rel_rms(_np(dv)[a:b][:, 1], rv[:, 1]), dg=rel_rms(_np(dg)[a:b][:, hs], rg[:, hs]))
    # dsink from its definition with the forward oracle's o and lse (all sequences)
    qh = x.q[:, 4:8].contiguous()
    fo, fl = oracle.forward(qh, x.k[:, 1:2].contiguous(), x.v[:, 1:2].contiguous(), x.cu_seqlens, x.scale, 0,
                            x.sink[4:8], x.g[:, 4:8].contiguous())
    D = np.sum(fo * _np(x.do[:, 4:8]), axis=2)
    rs = -np.sum(np.exp(_np(x.sink[4:8])[None, :] - fl) * D, axis=0)
    errs["dsink"] = rel_rms(_np(ds)[4:8], rs)
    _say("   ", {k: f"{v:.3e}" for k, v in errs.items()})
    assert max(errs.values()) <= TOL
