"""Pins for the decode / split-K oracle against things other than itself.

  * fp8 e4m3fn decoding: the oracle's own bit formula against torch's
    float8_e4m3fn -> float conversion on all 256 codes, plus values fixed by
    the OCP format (largest finite 448, the two NaN codes, subnormals);
  * paged decode on the dequantised cache = the prefill oracle's last n rows
    on the same keys and values laid out densely (cross-pin of two code
    paths written independently);
  * a permuted page table gives the same output;
  * split invariance: any segmentation merged by the reduce gives the
    unsplit result; empty partials change nothing; one partial gives acc / l;
    S identical partials give acc / l;
  * NaN in unused scale slots and unused cache bytes never reach the result.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.util import rel_rms


def test_fp8_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])


def test_fp8_format_fixed_points():
    f = oracle.fp8_e4m3fn_to_f64
    assert f(0x7E) == 448.0 and f(0xFE) == -448.0
    assert np.isnan(f(0x7F)) and np.isnan(f(0xFF))
    assert f(0x38) == 1.0 and f(0x08) == 2.0 ** -6
    assert f(0x01) == 2.0 ** -9 and f(0x07) == 7 * 2.0 ** -9
    assert f(0x00) == 0.0 and f(0x80) == 0.0


def _dense_forward_of_request(d, r):
    """Dequantise request r's K/V and run the prefill oracle over it; the
    last q_len rows of that run are the decode outputs."""
    L = int(d.seq_lens[r]); n = d.q_lens[r]
    fp8 = d.kv_dtype == synth.KV_FP8_E4M3FN
    kc = d.k_cache.numpy() if fp8 else d.k_cache
    vc = d.v_cache.numpy() if fp8 else d.v_cache
    K = oracle.gather_request_kv(kc if fp8 else kc.double().numpy(), d.k_scale,
                                 d.block_table, r, L, d.block_size, fp8)
    V = oracle.gather_request_kv(vc if fp8 else vc.double().numpy(), d.v_scale,
                                 d.block_table, r, L, d.block_size, fp8)
    Hq = d.q.shape[1]
    q = np.zeros((L, Hq, d.q.shape[2]))
    a = int(d.cu_seqlens_q[r])
    q[L - n:] = d.q[a:a + n].double().numpy()
    o, lse = oracle.forward(q, K, V, np.array([0, L]), d.scale)
    return o[L - n:], lse[L - n:]


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_FP8_E4M3FN], ids=["bf16", "fp8"])
@pytest.mark.parametrize("B", [16, 128])
def test_decode_equals_prefill_rows_on_dequantised_cache(kv, B):
    d = synth.decode_inputs([1, 37, 300, 129], [1, 4, 2, 3], 8, 2, 16, B,
                            kv_dtype=kv, seed=7, spare_pages=3)
    o, lse = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache,
                                 d.block_table, d.seq_lens, d.scale,
                                 kv == synth.KV_FP8_E4M3FN, d.k_scale, d.v_scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for r in range(4):
        a, b = int(d.cu_seqlens_q[r]), int(d.cu_seqlens_q[r + 1])
        ro, rl = _dense_forward_of_request(d, r)
        np.testing.assert_allclose(o[a:b], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[a:b], rl, rtol=1e-12)


def test_page_table_permutation_invariance():
    d = synth.decode_inputs([70, 33], [2, 1], 4, 1, 8, 16, kv_dtype=synth.KV_FP8_E4M3FN,
                            seed=3, spare_pages=5)
    fp8 = True
    o1, _ = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache,
                                d.block_table, d.seq_lens, d.scale, fp8, d.k_scale, d.v_scale)
    # move every page to a new id
    NB = d.num_blocks
    perm = np.random.default_rng(0).permutation(NB)
    kc = np.empty_like(d.k_cache.numpy()); vc = np.empty_like(d.v_cache.numpy())
    ks = np.empty_like(d.k_scale.numpy()); vs = np.empty_like(d.v_scale.numpy())
    kc[perm] = d.k_cache.numpy(); vc[perm] = d.v_cache.numpy()
    ks[perm] = d.k_scale.numpy(); vs[perm] = d.v_scale.numpy()
    bt = perm[d.block_table.numpy()]
    o2, _ = oracle.decode_paged(d.q, d.cu_seqlens_q, kc, vc, bt, d.seq_lens, d.scale,
                                fp8, ks, vs)
    np.testing.assert_array_equal(o1, o2)


def test_unused_slots_are_poisoned_and_ignored():
    d = synth.decode_inputs([20], [1], 2, 1, 8, 16, kv_dtype=synth.KV_FP8_E4M3FN,
                            seed=1, spare_pages=2)
    page = int(d.block_table[0, 1])
    assert np.isnan(d.k_scale[page, 0, 4:].numpy()).all()
    assert (d.k_cache[page, 0, 4:].numpy() == synth.FP8_POISON_BYTE).all()
    o, _ = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache,
                               d.block_table, d.seq_lens, d.scale, True, d.k_scale, d.v_scale)
    assert np.isfinite(o).all()


@pytest.mark.parametrize("split_len", [16, 48, 64, 1000])
def test_split_invariance(split_len):
    d = synth.decode_inputs([1, 5, 100, 257], [1, 4, 3, 4], 8, 2, 16, 16,
                            kv_dtype=synth.KV_FP8_E4M3FN, seed=17, spare_pages=1)
    args = (d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
            d.scale, True)
    o, lse = oracle.decode_paged(*args, d.k_scale, d.v_scale)
    S = math.ceil(d.max_seq_len / split_len)
    acc, m, l = oracle.decode_partials(*args, split_len, S, d.k_scale, d.v_scale)
    ro, rl = oracle.splitk_reduce(acc, m, l)
    np.testing.assert_allclose(ro.reshape(o.shape), o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rl.reshape(lse.shape), lse, rtol=1e-12)
    # short requests leave trailing splits empty, with m = -inf and l = 0
    assert np.isneginf(m).any() == (S > 1)


def test_empty_partial_for_query_ending_before_segment():
    """A 4-token verify whose first query sits just before a segment
    boundary: that query's partial for the next segment is empty."""
    d = synth.decode_inputs([35], [4], 2, 1, 8, 16, kv_dtype=synth.KV_BF16, seed=2,
                            spare_pages=1)
    # queries at positions 31..34; split 32 -> query 0 (pos 31) sees only split 0
    acc, m, l = oracle.decode_partials(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache,
                                       d.block_table, d.seq_lens, d.scale, False, 32, 2)
    assert np.isneginf(m[0:2, 1]).all() and (l[0:2, 1] == 0).all()
    assert np.isfinite(m[2:, 1]).all()


def test_reduce_special_cases():
    rng = np.random.default_rng(0)
    acc = rng.standard_normal((5, 1, 7)); m = rng.standard_normal((5, 1))
    l = rng.random((5, 1)) + 0.5
    o, lse = oracle.splitk_reduce(acc, m, l)
    np.testing.assert_allclose(o, acc[:, 0] / l, rtol=1e-15)
    np.testing.assert_allclose(lse, m[:, 0] + np.log(l[:, 0]), rtol=1e-15)
    # S identical partials: o = acc / l, lse = m + ln(S l)
    S = 6
    o2, lse2 = oracle.splitk_reduce(np.repeat(acc, S, 1), np.repeat(m, S, 1),
                                    np.repeat(l, S, 1))
    np.testing.assert_allclose(o2, acc[:, 0] / l, rtol=1e-14)
    np.testing.assert_allclose(lse2, m[:, 0] + np.log(S * l[:, 0]), rtol=1e-14)
    # adding empty partials (poisoned acc / l) changes nothing
    acc3 = np.concatenate([acc, np.full((5, 2, 7), np.nan)], 1)
    m3 = np.concatenate([m, np.full((5, 2), -np.inf)], 1)
    l3 = np.concatenate([l, np.full((5, 2), np.nan)], 1)
    o3, lse3 = oracle.splitk_reduce(acc3, m3, l3)
    np.testing.assert_array_equal(o3, o); np.testing.assert_array_equal(lse3, lse)
    # all empty: o = 0, lse = -inf
    o4, lse4 = oracle.splitk_reduce(acc3[:, 1:], m3[:, 1:], l3[:, 1:])
    assert (o4 == 0).all() and np.isneginf(lse4).all()


def test_reduce_of_split_softmax_equals_softmax():
    """Brute force: a softmax over 40 logits split into uneven pieces."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(40) * 5
    V = rng.standard_normal((40, 3))
    cuts = [0, 3, 4, 20, 40]
    acc = np.zeros((1, 4, 3)); m = np.zeros((1, 4)); l = np.zeros((1, 4))
    for s in range(4):
        xs = x[cuts[s]:cuts[s + 1]]
        m[0, s] = xs.max(); e = np.exp(xs - xs.max())
        l[0, s] = e.sum(); acc[0, s] = e @ V[cuts[s]:cuts[s + 1]]
    o, lse = oracle.splitk_reduce(acc, m, l)
    p = np.exp(x - x.max()); p /= p.sum()
    np.testing.assert_allclose(o[0], p @ V, rtol=1e-13)
    np.testing.assert_allclose(lse[0], np.log(np.sum(np.exp(x))), rtol=1e-13)


def test_quantised_cache_close_to_unquantised():
    """Diagnostic, not a pin: per-token fp8 with amax/448 scales stays within
    a few percent of the unquantised values and keeps token magnitudes."""
    d = synth.decode_inputs([200], [1], 4, 1, 64, 16, kv_dtype=synth.KV_FP8_E4M3FN,
                            seed=5, spare_pages=1, keep_unquantized=True)
    K = oracle.gather_request_kv(d.k_cache.numpy(), d.k_scale, d.block_table, 0, 200, 16, True)
    bt = d.block_table.numpy()[0]
    j = np.arange(200)
    X = d.unquantized_k.numpy()[bt[j // 16], :, j % 16, :]
    assert rel_rms(K, X) < 0.05


# ----------------------------------------------------------------------------
# decode with sink, sliding window, log gate and per-tensor scales
# ----------------------------------------------------------------------------
def _dense_request(d, r, fp8=True):
    B = d.block_size
    L = int(d.seq_lens[r])
    host = lambda c: c.double().numpy() if c.dtype == torch.bfloat16 else c.numpy()
    K = oracle.gather_request_kv(host(d.k_cache), None if d.k_scale is None else d.k_scale.numpy(),
                                 d.block_table.numpy(), r, L, B, fp8, d.per_tensor)
    V = oracle.gather_request_kv(host(d.v_cache), None if d.v_scale is None else d.v_scale.numpy(),
                                 d.block_table.numpy(), r, L, B, fp8, d.per_tensor)
    return K, V


@pytest.mark.parametrize("window,sink,gate", [(0, True, False), (48, False, False), (0, False, True),
                                              (100, True, True), (1, True, True)])
def test_decode_features_equal_prefill_rows(window, sink, gate):
    """Decode with sink / window / gate on the dequantised cache equals the
    prefill oracle's rows for the same query positions, with the gates given
    as differences of the cached cumulative gate."""
    d = synth.decode_inputs([70, 260], [1, 3], 8, 2, 64, 16, kv_dtype=synth.KV_FP8_E4M3FN, seed=21,
                            window=window, with_sink=sink, with_gate=gate, spare_pages=2)
    o, lse = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, True, d.k_scale, d.v_scale, sink=d.sink, window=d.window,
                                 g_cache=d.g_cache)
    cu = d.cu_seqlens_q.numpy()
    for r in range(2):
        L = int(d.seq_lens[r]); n = int(cu[r + 1] - cu[r])
        K, V = _dense_request(d, r)
        q = np.zeros((L, 8, 64)); q[L - n:] = d.q[cu[r]:cu[r + 1]].double().numpy()
        g = None
        if gate:
            G = oracle.gather_request_gates(d.g_cache.numpy(), d.block_table.numpy(), r, L, d.block_size)
            g = np.diff(np.concatenate([np.zeros((1, 8)), G]), axis=0)
        ro, rl = oracle.forward_rows(q, K, V, np.array([0, L]), d.scale, list(range(L - n, L)),
                                     list(range(8)), window=window, sink=d.sink, g=g)
        np.testing.assert_allclose(o[cu[r]:cu[r + 1]], ro, rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(lse[cu[r]:cu[r + 1]], rl, rtol=1e-9, atol=1e-9)


def test_decode_window_one_closed_form():
    """Window 1: the query sees only its own key, so o = v_p e^s / (e^s + e^sink)."""
    d = synth.decode_inputs([33], [2], 4, 1, 64, 16, kv_dtype=synth.KV_BF16, seed=22, window=1,
                            with_sink=True, spare_pages=1)
    o, _ = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                               d.scale, False, sink=d.sink, window=1)
    K, V = _dense_request(d, 0, fp8=False)
    for t, p in enumerate((31, 32)):
        for h in range(4):
            s = d.scale * float(K[p, 0] @ d.q[t, h].double().numpy())
            w = np.exp(s) / (np.exp(s) + np.exp(float(d.sink[h])))
            np.testing.assert_allclose(o[t, h], w * V[p, 0], rtol=1e-12, atol=1e-12)


def test_per_tensor_scales_equal_uniform_per_token_scales():
    d = synth.decode_inputs([50, 90], [1, 2], 8, 2, 64, 16, kv_dtype=synth.KV_FP8_E4M3FN, seed=23,
                            per_tensor=True, spare_pages=1)
    o1, l1 = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, True, d.k_scale, d.v_scale, per_tensor=True)
    NB, Hkv, B = d.k_cache.shape[:3]
    ks = np.full((NB, Hkv, B), float(d.k_scale[0])); vs = np.full((NB, Hkv, B), float(d.v_scale[0]))
    o2, l2 = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, True, ks, vs)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_split_invariance_with_sink_window_gate():
    d = synth.decode_inputs([70, 260], [1, 3], 8, 2, 64, 16, kv_dtype=synth.KV_FP8_E4M3FN, seed=24,
                            window=40, with_sink=True, with_gate=True, spare_pages=2)
    o, lse = oracle.decode_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 d.scale, True, d.k_scale, d.v_scale, sink=d.sink, window=d.window,
                                 g_cache=d.g_cache)
    for split in (16, 32, 64):
        S = (260 + split - 1) // split
        acc, m, l = oracle.decode_partials(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table,
                                           d.seq_lens, d.scale, True, split, S, d.k_scale, d.v_scale,
                                           sink=d.sink, window=d.window, g_cache=d.g_cache)
        ro, rl = oracle.splitk_reduce(acc, m, l)
        np.testing.assert_allclose(ro.reshape(o.shape), o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rl.reshape(lse.shape), lse, rtol=1e-10, atol=1e-12)
