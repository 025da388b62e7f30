"""GPU parity of the HIP path against the float64 oracle on small inputs that
still span several tiles and end in ragged tails.

Bars: relative RMS error <= 5e-3 for outputs and every gradient (the
tolerance the fla issue #1322 sink-gradient comment measures against), and
<= 1e-6 for the fp32 split-K merge of identical partials.
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
    sys.stdout.flush()


@pytest.fixture(scope="module")
def A():
    import causal_softmax_attention_amd as A
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return A


def _np(t):
    return t.detach().float().cpu().double().numpy()


# ----------------------------------------------------------------------------
# split-K reduce
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dv", [64, 128, 512])
@pytest.mark.parametrize("S", [1, 3, 8, 17])
def test_splitk_reduce_random_partials(A, dv, S):
    _say(f"[case] splitk_reduce dv={dv} S={S}")
    acc, m, l = synth.partials_inputs(301, S, dv, seed=S * 7 + dv, device=DEV)
    out, lse = A.attn_splitk_reduce(acc, m, l, torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.splitk_reduce(acc.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy())
    assert rel_rms(_np(out), ro) <= 1e-6
    assert np.max(np.abs(_np(lse) - rl)) <= 1e-5
    outb, _ = A.attn_splitk_reduce(acc, m, l, torch.bfloat16, return_lse=False)
    assert rel_rms(_np(outb), ro) <= TOL


def test_splitk_reduce_identical_partials(A):
    _say("[case] splitk_reduce identical partials")
    acc1, m1, l1 = synth.partials_inputs(257, 1, 128, seed=5, empty_frac=0.0, device=DEV)
    S = 9
    acc = acc1.repeat(1, S, 1).contiguous()
    m = m1.repeat(1, S).contiguous()
    l = l1.repeat(1, S).contiguous()
    out, lse = A.attn_splitk_reduce(acc, m, l, torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.splitk_reduce(acc.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy())
    assert rel_rms(_np(out), ro) <= 1e-6
    np.testing.assert_allclose(_np(out), (acc1[:, 0] / l1).cpu().double().numpy(), rtol=1e-5, atol=1e-6)
    assert np.max(np.abs(_np(lse) - rl)) <= 1e-5


def test_splitk_reduce_all_empty_rows(A):
    _say("[case] splitk_reduce all-empty rows")
    acc, m, l = synth.partials_inputs(64, 4, 64, seed=9, empty_frac=1.0, device=DEV)
    out, lse = A.attn_splitk_reduce(acc, m, l, torch.float32)
    torch.cuda.synchronize()
    assert (out == 0).all().item()
    assert torch.isneginf(lse).all().item()


# ----------------------------------------------------------------------------
# paged decode
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # seq_lens, q_lens, Hq, Hkv, D, B, kv
    ([1, 37, 300, 1029, 4096], [1, 1, 1, 1, 1], 64, 4, 128, 16, synth.KV_FP8_E4M3FN),
    ([1, 37, 300, 1029, 4096], [1, 1, 1, 1, 1], 64, 4, 128, 16, synth.KV_BF16),
    ([5, 130, 2051, 4000], [4, 2, 3, 4], 64, 4, 128, 128, synth.KV_FP8_E4M3FN),
    ([5, 130, 2051, 4000], [4, 2, 3, 4], 64, 4, 128, 128, synth.KV_BF16),
    ([17, 700, 2500], [1, 1, 1], 16, 2, 128, 16, synth.KV_FP8_E4M3FN),      # GQA 8
    ([17, 700, 2500], [2, 4, 1], 8, 8, 64, 32, synth.KV_BF16),              # MHA, D 64
    ([64, 65537], [4, 4], 32, 2, 128, 64, synth.KV_BF16),             # the aiter PR's Test plan context
    ([1, 37, 300, 1029, 4096], [1, 1, 1, 1, 1], 32, 4, 64, 16, synth.KV_FP8_E4M3FN),   # fp8, D 64
    ([5, 130, 2051], [4, 2, 3], 16, 4, 64, 64, synth.KV_FP8_E4M3FN),   # fp8, D 64, short queries
    ([5, 130, 2051], [4, 2, 3], 64, 4, 64, 64, synth.KV_FP8_E4M3FN),   # fp8, D 64, two-wave verify shape
]


def _decode_ids(c):
    return f"L{max(c[0])}-q{max(c[1])}-h{c[2]}kv{c[3]}-d{c[4]}-p{c[5]}-{'fp8' if c[6] else 'bf16'}"


@pytest.mark.parametrize("case", DECODE_CASES, ids=_decode_ids)
def test_decode_matches_oracle(A, case):
    seq_lens, q_lens, Hq, Hkv, D, B, kv = case
    _say(f"[case] decode {_decode_ids(case)}")
    d = synth.decode_inputs(seq_lens, q_lens, Hq, Hkv, D, B, kv_dtype=kv, seed=len(seq_lens) + D + B,
                            device=DEV, spare_pages=5)
    out, lse = A.attn_decode_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, kv,
                                   d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len,
                                   d.scale, return_lse=True)
    torch.cuda.synchronize()
    fp8 = kv == synth.KV_FP8_E4M3FN
    ro, rl = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, fp8, d.k_scale, d.v_scale)
    o = _np(out)
    assert np.isfinite(o).all()
    err = rel_rms(o, ro)
    bias = float(np.sum(o * ro) / np.sum(ro * ro) - 1.0)
    _say(f"    rel_rms={err:.3e} bias={bias:.2e}")
    assert err <= TOL
    assert abs(bias) < 1e-3
    assert np.max(np.abs(_np(lse) - rl)) <= 1e-3


BALANCED_CASES = [
    # seq_lens, q_lens, Hq, Hkv, D, B, kv, sink, gate, per-tensor
    ([1, 2, 3, 40, 5000, 7, 31, 32, 33, 900], [1] * 10, 64, 4, 128, 16, synth.KV_FP8_E4M3FN, False, False, False),
    ([3000, 17, 64, 2049, 4], [4, 3, 1, 2, 4], 64, 4, 128, 16, synth.KV_FP8_E4M3FN, True, True, False),
    ([129, 4100, 1, 600], [2, 1, 1, 4], 16, 2, 64, 32, synth.KV_BF16, True, False, False),
    ([6000, 6000, 5], [1, 4, 1], 64, 4, 128, 128, synth.KV_FP8_E4M3FN, False, True, True),
    ([2, 900, 3100, 45], [1, 1, 4, 2], 32, 4, 64, 16, synth.KV_FP8_E4M3FN, True, True, False),
]


def _bal_id(c):
    L, q, Hq, Hkv, D, B, kv, sk, gt, pt = c
    return (f"r{len(L)}-L{max(L)}-q{max(q)}-h{Hq}kv{Hkv}-d{D}-p{B}-{'fp8' if kv else 'bf16'}"
            f"{'-sink' if sk else ''}{'-gate' if gt else ''}{'-pt' if pt else ''}")


@pytest.mark.parametrize("case", BALANCED_CASES, ids=_bal_id)
def test_decode_balanced_split(A, case):
    """The library's split of a decode without a window gives every
    workgroup an equal share of all keys (pieces that cross requests and
    start or end mid-step); it matches the oracle and the fixed-length
    split."""
    L, q, Hq, Hkv, D, B, kv, sk, gt, pt = case
    _say(f"[case] decode balanced {_bal_id(case)}")
    d = synth.decode_inputs(L, q, Hq, Hkv, D, B, kv_dtype=kv, seed=sum(L) % 1000, device=DEV,
                            with_sink=sk, with_gate=gt, per_tensor=pt, spare_pages=4)
    args = (d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype, d.k_scale, d.v_scale,
            d.block_table, d.seq_lens, d.max_seq_len, d.scale)
    kw = dict(return_lse=True, sink=d.sink, g_cache=d.g_cache)
    out, lse = A.attn_decode_paged(*args, **kw)
    fix_o, fix_l = A.attn_decode_paged(*args, kv_split_len=B if B > 32 else 256, **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, kv == synth.KV_FP8_E4M3FN, d.k_scale, d.v_scale, sink=d.sink,
                                 g_cache=d.g_cache, per_tensor=d.per_tensor)
    o = _np(out)
    assert np.isfinite(o).all()
    err = rel_rms(o, ro)
    lerr = float(np.max(np.abs(_np(lse) - rl)))
    _say(f"    rel_rms={err:.3e} lse max abs={lerr:.2e} vs fixed split {rel_rms(o, _np(fix_o)):.2e}")
    assert err <= TOL
    assert lerr <= 1e-3
    assert rel_rms(o, _np(fix_o)) <= 2e-3
    assert float(np.max(np.abs(_np(lse) - _np(fix_l)))) <= 1e-4


@pytest.mark.parametrize("split", [32, 128, 512, 2048])
def test_decode_split_invariance(A, split):
    _say(f"[case] decode split={split}")
    d = synth.decode_inputs([33, 1000, 3000], [4, 1, 3], 64, 4, 128, 32, kv_dtype=synth.KV_FP8_E4M3FN,
                            seed=77, device=DEV, spare_pages=3)
    args = (d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype, d.k_scale,
            d.v_scale, d.block_table, d.seq_lens, d.max_seq_len, d.scale)
    out = A.attn_decode_paged(*args, kv_split_len=split)
    torch.cuda.synchronize()
    ro, _ = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                d.scale, True, d.k_scale, d.v_scale)
    assert rel_rms(_np(out), ro) <= TOL


def test_decode_nan_poison_never_leaks(A):
    """Unused scale slots are NaN and unused cache bytes a NaN code; a
    request whose length is an exact page multiple, and one ending one token
    into a page, must both stay finite."""
    _say("[case] decode NaN poison")
    d = synth.decode_inputs([16, 17, 31, 32, 33], [1, 1, 2, 3, 4], 64, 4, 128, 16,
                            kv_dtype=synth.KV_FP8_E4M3FN, seed=3, device=DEV, spare_pages=2)
    out = A.attn_decode_paged(d.q, d.cu_seqlens_q, 4, d.k_cache, d.v_cache, d.kv_dtype, d.k_scale,
                              d.v_scale, d.block_table, d.seq_lens, 33, d.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()


# ----------------------------------------------------------------------------
# prefill forward / backward
# ----------------------------------------------------------------------------
PREFILL_CASES = [
    # seqlens, Hq, Hkv, dqk, dv, window, sink, gate
    ([128], 4, 1, 64, 64, 0, True, False),
    ([1, 77, 300, 129], 8, 2, 64, 64, 0, True, True),
    ([5, 333, 700], 8, 2, 128, 128, 100, True, True),
    ([700, 64, 1], 4, 4, 128, 128, 0, False, False),
    ([260, 97], 4, 1, 128, 128, 37, False, True),
    ([300, 190], 4, 2, 256, 256, 0, True, True),
    ([257, 130], 4, 1, 256, 512, 0, True, True),
    ([257, 130], 4, 2, 256, 512, 64, True, False),
    # unequal query/key and value head dims: every pair of d_qk in {64, 128, 256}
    # and d_v in {64, 128, 256, 512} not covered above
    ([3, 190, 77], 8, 2, 64, 128, 0, True, True),
    ([150, 61], 4, 4, 128, 64, 50, True, False),
    ([1, 140, 97], 4, 1, 64, 256, 0, True, True),
    ([129, 70], 4, 2, 64, 512, 40, False, True),
    ([200, 33], 8, 2, 128, 256, 0, True, True),
    ([97, 160], 4, 1, 128, 512, 0, True, False),
    ([180, 45], 4, 2, 256, 64, 0, True, True),
    ([77, 150], 8, 2, 256, 128, 60, False, True),
    # one query head per workgroup in the large-head kernels: MHA, and a KV
    # group of three heads
    ([200, 37], 4, 4, 256, 512, 0, True, True),
    ([150, 90], 6, 2, 128, 256, 50, True, True),
    # the backward's dS store over many row tiles and key-block slots: a
    # window band of 300 keys, and an unwindowed causal triangle
    ([1500, 700], 4, 2, 256, 512, 300, True, True),
    ([2100], 4, 1, 128, 512, 0, True, True),
]


def _pf_id(c):
    s, Hq, Hkv, dqk, dv, W, sk, gt = c
    return f"T{sum(s)}n{len(s)}-h{Hq}kv{Hkv}-d{dqk}x{dv}-w{W}{'-sink' if sk else ''}{'-gate' if gt else ''}"


def _prefill(c, seed):
    s, Hq, Hkv, dqk, dv, W, sk, gt = c
    return synth.prefill_inputs(s, Hq, Hkv, dqk, dv, seed=seed, window=W, with_sink=sk,
                                with_gate=gt, device=DEV)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=_pf_id)
def test_forward_matches_oracle(A, case):
    _say(f"[case] forward {_pf_id(case)}")
    x = _prefill(case, seed=123)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window,
                               x.sink, x.g)
    torch.cuda.synchronize()
    ro, rl = oracle.forward(x.q, x.k, x.v, x.cu_seqlens, x.scale, x.window, x.sink, x.g)
    err = rel_rms(_np(o), ro)
    _say(f"    o rel_rms={err:.3e} lse max abs={np.max(np.abs(_np(lse) - rl)):.2e}")
    assert err <= TOL
    assert np.max(np.abs(_np(lse) - rl)) <= 2e-3


# two-pass with the dS store (the default), two-pass recomputing S and dP in
# the dQ pass, fused dQ; the fused-dQ backward covers d_qk <= 128 (larger
# heads are rejected, see test_fused_dq_rejects_large_heads)
BACKWARD_CASES = [(c, m) for c in PREFILL_CASES for m in ("two-pass", "recompute-dq", "fused-dq")
                  if not (m == "fused-dq" and c[3] > 128)]
BWD_FLAGS = {"two-pass": 0, "recompute-dq": 4, "fused-dq": 2}


@pytest.mark.parametrize("case,mode", BACKWARD_CASES, ids=lambda v: v if isinstance(v, str) else _pf_id(v))
def test_backward_matches_oracle(A, case, mode):
    flags = BWD_FLAGS[mode]
    _say(f"[case] backward {mode} {_pf_id(case)}")
    x = _prefill(case, seed=321)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window,
                               x.sink, x.g)
    dq, dk, dv, ds, dg = A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen,
                                           x.scale, x.window, x.sink, x.g, flags=flags)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.do, x.cu_seqlens, x.scale, x.window, x.sink, x.g)
    names = ["dq", "dk", "dv", "dsink", "dg"]
    errs = {}
    for nm, got, want in zip(names, (dq, dk, dv, ds, dg), ref):
        if want is None:
            assert got is None
            continue
        errs[nm] = rel_rms(_np(got), want)
    _say("    " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for nm, e in errs.items():
        assert e <= TOL, nm


# flags 1 stores dS between the passes for the large heads (case 5: d 256 x
# 256) and recomputes for the others (case 2: d 128); flags 5 always recomputes
@pytest.mark.parametrize("ci,flags", [(2, 1), (5, 1), (5, 5)], ids=["d128", "d256-ds-store", "d256-recompute"])
def test_backward_two_pass_is_bitwise_deterministic(A, ci, flags):
    _say(f"[case] backward determinism case {ci} flags={flags}")
    x = _prefill(PREFILL_CASES[ci], seed=9)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window, x.sink, x.g)
    runs = [A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale, x.window,
                              x.sink, x.g, flags=flags) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_fused_dq_rejects_large_heads(A):
    x = _prefill(next(c for c in PREFILL_CASES if c[3] == 256), seed=1)   # d_qk 256
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window, x.sink, x.g)
    with pytest.raises(NotImplementedError, match="fused-dQ"):
        A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale, x.window,
                          x.sink, x.g, flags=A.ATTN_BWD_FUSED_DQ)


def test_forward_empty_and_zero_length_sequences(A):
    _say("[case] forward with zero-length sequences")
    x = synth.prefill_inputs([0, 40, 0, 3], 4, 2, 64, 64, seed=4, window=0, device=DEV)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, 0, x.sink, x.g)
    torch.cuda.synchronize()
    ro, _ = oracle.forward(x.q, x.k, x.v, x.cu_seqlens, x.scale, 0, x.sink, x.g)
    assert rel_rms(_np(o), ro) <= TOL


# zero-length sequences around short ones, through both backward paths: the
# dS store (d 128 x 512, d 256 x 512) and the recomputing dQ pass (d 64 x 64)
@pytest.mark.parametrize("dqk,dv,W", [(64, 64, 0), (128, 512, 0), (256, 512, 20)])
def test_backward_zero_length_sequences(A, dqk, dv, W):
    _say(f"[case] backward with zero-length sequences d{dqk}x{dv} w{W}")
    x = synth.prefill_inputs([0, 40, 0, 3, 70, 0], 4, 2, dqk, dv, seed=6, window=W, device=DEV)
    o, lse = A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, W, x.sink, x.g)
    got = A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale, W, x.sink, x.g)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.do, x.cu_seqlens, x.scale, W, x.sink, x.g)
    errs = {nm: rel_rms(_np(gt), want) for nm, gt, want in zip(["dq", "dk", "dv", "dsink", "dg"], got, ref)}
    _say("    " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL


# ----------------------------------------------------------------------------
# decode with sink / sliding window / log gate / per-tensor scales
# ----------------------------------------------------------------------------
FEATURE_CASES = [
    # seq_lens, q_lens, Hq, Hkv, D, B, kv, window, sink, gate, per_tensor, split
    ([40, 700, 2500], [1, 1, 1], 64, 4, 128, 16, synth.KV_FP8_E4M3FN, 0, True, False, False, 0),
    ([40, 700, 2500], [1, 2, 4], 16, 4, 128, 16, synth.KV_FP8_E4M3FN, 300, False, False, False, 256),
    ([40, 700, 2500], [1, 1, 3], 32, 2, 128, 32, synth.KV_FP8_E4M3FN, 0, False, True, False, 512),
    ([5, 900, 4100], [4, 2, 3], 64, 4, 128, 128, synth.KV_FP8_E4M3FN, 1000, True, True, False, 0),
    ([5, 900, 4100], [4, 2, 3], 64, 4, 128, 16, synth.KV_FP8_E4M3FN, 77, True, True, True, 1024),
    ([33, 1500], [2, 1], 8, 8, 64, 32, synth.KV_BF16, 200, True, True, False, 256),
    ([33, 1500], [2, 4], 32, 4, 128, 64, synth.KV_BF16, 0, True, True, False, 0),
    ([6000], [4], 64, 4, 128, 16, synth.KV_FP8_E4M3FN, 1, True, False, True, 512),
]


def _feat_id(c):
    L, ql, Hq, Hkv, D, B, kv, W, sk, gt, pt, sp = c
    return (f"L{max(L)}-q{max(ql)}-h{Hq}kv{Hkv}-d{D}-p{B}-{'fp8' if kv else 'bf16'}-w{W}"
            f"{'-sink' if sk else ''}{'-gate' if gt else ''}{'-pt' if pt else ''}-s{sp}")


@pytest.mark.parametrize("case", FEATURE_CASES, ids=_feat_id)
def test_decode_features_match_oracle(A, case):
    L, ql, Hq, Hkv, D, B, kv, W, sk, gt, pt, sp = case
    _say(f"[case] decode features {_feat_id(case)}")
    d = synth.decode_inputs(L, ql, Hq, Hkv, D, B, kv_dtype=kv, seed=sum(L) + Hq, device=DEV,
                            window=W, with_sink=sk, with_gate=gt, per_tensor=pt, spare_pages=4)
    fp8 = kv == synth.KV_FP8_E4M3FN
    out, lse = A.attn_decode_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype,
                                   d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len, d.scale,
                                   kv_split_len=sp, return_lse=True, sink=d.sink, window=d.window,
                                   g_cache=d.g_cache)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, fp8, d.k_scale, d.v_scale, sink=d.sink, window=d.window,
                                 g_cache=d.g_cache, per_tensor=d.per_tensor)
    o = _np(out)
    assert np.isfinite(o).all()
    err = rel_rms(o, ro)
    bias = float(np.sum(o * ro) / np.sum(ro * ro) - 1.0)
    lerr = float(np.max(np.abs(_np(lse) - rl)))
    _say(f"    rel_rms={err:.3e} bias={bias:.2e} lse max abs={lerr:.2e}")
    assert err <= TOL
    assert abs(bias) < 1e-3
    assert lerr <= 1e-3
