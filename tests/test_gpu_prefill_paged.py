"""GPU parity of the paged prefill (any number of new tokens per request over
the paged bf16 / per-token fp8 cache) against the float64 oracle.

Small cases compare every output element (relative RMS <= 5e-3, the bar of
the rest of the path; lse max abs <= 1e-3; output bias below 1e-3) and span
several 128-row query blocks, ragged last blocks, single-segment (direct
output) and split-K launches, mixed batches with decode rows, GQA 16 / 4 / 1,
head dim 64 and 128, and the sink / window / gate / per-tensor-scale
features, on both kernels (the split-K kernel and, for single-segment
calls, the pipelined tile kernel).  The chunked-prefill workload the benchmark times is checked on
sampled rows against the prefill oracle's rows of the whole sequence.
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


FP8, BF16 = synth.KV_FP8_E4M3FN, synth.KV_BF16
# (seq_lens, new tokens, Hq, Hkv, D, page, kv, window, sink, gate, per-tensor, split)
CASES = [
    ([300, 1000, 77], [300, 129, 5], 64, 4, 128, 16, FP8, 0, False, False, False, 0),
    ([300, 1000, 77], [300, 129, 5], 64, 4, 128, 16, FP8, 0, False, False, False, 1024),
    ([90, 700, 260, 33], [1, 4, 70, 33], 32, 4, 128, 128, BF16, 100, True, True, False, 0),
    ([513, 2000], [513, 300], 8, 2, 64, 32, BF16, 0, True, False, False, 256),
    ([1, 4000], [1, 9], 64, 4, 128, 16, FP8, 0, False, True, True, 0),
    ([2500], [2500], 16, 16, 128, 64, FP8, 700, True, True, False, 0),
    ([600, 1500], [600, 200], 16, 4, 64, 32, FP8, 0, True, True, False, 0),      # fp8, D 64
    # one segment per query tile on an fp8 cache without a gate: the
    # pipelined tile kernel (GQA 16 / 8 / 2 / 1, ragged tiles, window, sink,
    # per-tensor scales, pages of 16 / 32 / 64 keys, D 64 and 128)
    ([1200, 700], [1200, 300], 64, 4, 128, 16, FP8, 0, False, False, False, 65536),
    ([900, 2000], [900, 129], 16, 8, 128, 32, FP8, 300, True, False, False, 65536),
    ([1000, 50], [100, 50], 32, 4, 128, 64, FP8, 0, True, False, True, 65536),
    ([600], [400], 4, 4, 64, 16, FP8, 0, True, False, True, 65536),
    ([700, 333], [700, 333], 16, 4, 64, 16, FP8, 200, False, False, False, 65536),
    # the same kernel on a bf16 cache and with the gate cache
    ([800, 1600], [800, 300], 32, 4, 128, 16, BF16, 200, True, False, False, 65536),
    ([700], [700], 8, 4, 64, 32, BF16, 0, False, True, False, 65536),
    ([900, 400], [600, 400], 64, 4, 128, 16, FP8, 0, True, True, False, 65536),
    ([1000], [513], 16, 4, 128, 64, FP8, 300, False, True, True, 65536),
    ([2500], [2500], 16, 16, 128, 64, FP8, 700, True, True, False, 65536),
]


def _id(c):
    L, n, Hq, Hkv, D, B, kv, W, sk, gt, pt, sp = c
    return (f"L{max(L)}-n{max(n)}-r{len(L)}-h{Hq}kv{Hkv}-d{D}-p{B}-{'fp8' if kv else 'bf16'}-w{W}"
            f"{'-sink' if sk else ''}{'-gate' if gt else ''}{'-pt' if pt else ''}-s{sp}")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_prefill_paged_matches_oracle(A, case):
    L, n, Hq, Hkv, D, B, kv, W, sk, gt, pt, sp = case
    _say(f"[case] paged prefill {_id(case)}")
    d = synth.decode_inputs(L, n, Hq, Hkv, D, B, kv_dtype=kv, seed=sum(L) + 7 * Hq, device=DEV,
                            window=W, with_sink=sk, with_gate=gt, per_tensor=pt, spare_pages=4)
    out, lse = A.attn_prefill_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype,
                                    d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len, d.scale,
                                    kv_split_len=sp, return_lse=True, sink=d.sink, window=d.window,
                                    g_cache=d.g_cache)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                  d.scale, kv == FP8, d.k_scale, d.v_scale, sink=d.sink, window=d.window,
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


def test_prefill_paged_split_invariance(A):
    """Single-segment (direct output) and split-K launches agree."""
    _say("[case] paged prefill split invariance")
    d = synth.decode_inputs([700, 1500], [200, 64], 32, 4, 128, 16, kv_dtype=FP8, seed=5, device=DEV,
                            with_sink=True, spare_pages=2)
    outs = []
    for sp in (0, 256, 2048):
        o, l = A.attn_prefill_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype,
                                    d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len, d.scale,
                                    kv_split_len=sp, return_lse=True, sink=d.sink)
        outs.append((_np(o), _np(l)))
    for o, l in outs[1:]:
        assert rel_rms(o, outs[0][0]) < 2e-3
        assert np.max(np.abs(l - outs[0][1])) < 1e-4


def test_prefill_paged_equals_decode_for_short_queries(A):
    """Rows of at most four tokens give the same result through either entry."""
    _say("[case] paged prefill vs decode, q_len <= 4")
    d = synth.decode_inputs([50, 3000, 130], [1, 4, 2], 64, 4, 128, 16, kv_dtype=FP8, seed=6, device=DEV,
                            spare_pages=2)
    args = (d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype, d.k_scale, d.v_scale,
            d.block_table, d.seq_lens, d.max_seq_len, d.scale)
    o1 = A.attn_decode_paged(*args, kv_split_len=512)
    o2 = A.attn_prefill_paged(*args, kv_split_len=512)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_prefill_paged_bench_workload_sampled_rows(A):
    """The chunked-prefill workload the benchmark times, in its launch
    configuration: sampled rows against the prefill oracle's rows of the
    whole sequence on the dequantised cache."""
    _say("[case] paged prefill bench workload, sampled rows")
    d = synth.prefill_paged_bench(device=DEV)
    out, lse = A.attn_prefill_paged(d.q, d.cu_seqlens_q, d.max_seqlen_q, d.k_cache, d.v_cache, d.kv_dtype,
                                    d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.max_seq_len, d.scale,
                                    return_lse=True)
    torch.cuda.synchronize()
    o, l = _np(out), _np(lse)
    assert np.isfinite(o).all()
    rng = np.random.default_rng(0)
    cu = d.cu_seqlens_q.cpu().numpy()
    Hq, D = d.q.shape[1], d.q.shape[2]
    errs = []
    for r in range(len(d.q_lens)):
        L = int(d.seq_lens[r]); n = d.q_lens[r]
        K = oracle.gather_request_kv(d.k_cache.cpu().numpy(), d.k_scale.cpu().numpy(),
                                     d.block_table.cpu().numpy(), r, L, d.block_size, True)
        V = oracle.gather_request_kv(d.v_cache.cpu().numpy(), d.v_scale.cpu().numpy(),
                                     d.block_table.cpu().numpy(), r, L, d.block_size, True)
        q = np.zeros((L, Hq, D)); q[L - n:] = d.q[cu[r]:cu[r + 1]].double().cpu().numpy()
        ts = sorted(set([0, n - 1] + list(rng.integers(0, n, 3))))
        hs = sorted(set([0, Hq - 1] + list(rng.integers(0, Hq, 2))))
        ro, rl = oracle.forward_rows(q, K, V, np.array([0, L]), d.scale, [L - n + t for t in ts], hs)
        for i, t in enumerate(ts):
            for j, h in enumerate(hs):
                errs.append(np.linalg.norm(o[cu[r] + t, h] - ro[i, j]) / np.linalg.norm(ro[i, j]))
                assert abs(l[cu[r] + t, h] - rl[i, j]) <= 1e-3
    rms = float(np.sqrt(np.mean(np.square(errs))))
    _say(f"    sampled rows={len(errs)} rel_rms={rms:.3e}")
    assert rms <= TOL
