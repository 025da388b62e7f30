"""Pins for the paged-prefill oracle (any number of new tokens per request
over the paged bf16 / per-token fp8 cache) against things other than itself.

  * a fresh prefill (n = L) over a bf16 cache equals the packed varlen
    prefill oracle on the same tokens laid out densely, with sink, sliding
    window and log gates (cross-pin of two code paths written
    independently; the dense layout is rebuilt here from the page table);
  * a chunked prefill (n < L) over an fp8 cache equals the prefill oracle's
    last n rows of the whole sequence on the dequantised keys and values;
  * a mixed batch (decode rows and prefill chunks in one call) equals each
    request run on its own;
  * segment splits merged by the reduce give the unsplit result, also where
    most segments lie past the early rows of a long chunk.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _dense_kv(d, r):
    """Request r's keys and values [L, Hkv, D] in float64, read through the
    page table with torch indexing (independent of the oracle's gather)."""
    L = int(d.seq_lens[r]); B = d.block_size
    j = torch.arange(L)
    pages = d.block_table[r].long()[j // B]
    slots = j % B
    out = []
    for c, sc in ((d.k_cache, d.k_scale), (d.v_cache, d.v_scale)):
        x = c[pages, :, slots, :]                      # [L, Hkv, D]
        if d.kv_dtype == synth.KV_FP8_E4M3FN:
            x = x.view(torch.float8_e4m3fn).double()
            x = x * (sc.double().reshape(1, 1, 1) if d.per_tensor else sc[pages, :, slots].double()[..., None])
        else:
            x = x.double()
        out.append(x.numpy())
    return out


def _cumulative_to_log_gates(d, r, Hq):
    """Per-token log gates whose per-sequence prefix sums are the cached G."""
    L = int(d.seq_lens[r]); B = d.block_size
    j = torch.arange(L)
    G = d.g_cache[d.block_table[r].long()[j // B], :, j % B].double().numpy()   # [L, Hq]
    return np.diff(np.concatenate([np.zeros((1, Hq)), G]), axis=0)


@pytest.mark.parametrize("window,sink,gate", [(0, False, False), (0, True, True), (33, True, False),
                                              (17, False, True)])
def test_fresh_prefill_equals_packed_prefill(window, sink, gate):
    lens = [45, 130, 7]
    d = synth.decode_inputs(lens, lens, 8, 2, 32, 16, kv_dtype=synth.KV_BF16, seed=31, window=window,
                            with_sink=sink, with_gate=gate, spare_pages=2)
    o, lse = oracle.prefill_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                  d.scale, False, sink=d.sink, window=window, g_cache=d.g_cache)
    K = np.concatenate([_dense_kv(d, r)[0] for r in range(3)])
    V = np.concatenate([_dense_kv(d, r)[1] for r in range(3)])
    g = np.concatenate([_cumulative_to_log_gates(d, r, 8) for r in range(3)]) if gate else None
    cu = np.concatenate([[0], np.cumsum(lens)])
    ro, rl = oracle.forward(d.q.double().numpy(), K, V, cu, d.scale, window=window,
                            sink=None if d.sink is None else d.sink.double().numpy(), g=g)
    np.testing.assert_allclose(o, ro, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(lse, rl, rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("B", [16, 128])
def test_chunked_prefill_equals_last_rows_of_whole_sequence(B):
    lens, news = [300, 129, 40], [77, 5, 40]
    d = synth.decode_inputs(lens, news, 8, 2, 32, B, kv_dtype=synth.KV_FP8_E4M3FN, seed=32,
                            with_sink=True, spare_pages=2)
    o, lse = oracle.prefill_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                  d.scale, True, d.k_scale, d.v_scale, sink=d.sink)
    cu = d.cu_seqlens_q.numpy()
    for r, (L, n) in enumerate(zip(lens, news)):
        K, V = _dense_kv(d, r)
        q = np.zeros((L, 8, 32)); q[L - n:] = d.q[cu[r]:cu[r + 1]].double().numpy()
        ro, rl = oracle.forward(q, K, V, np.array([0, L]), d.scale, sink=d.sink.double().numpy())
        np.testing.assert_allclose(o[cu[r]:cu[r + 1]], ro[L - n:], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(lse[cu[r]:cu[r + 1]], rl[L - n:], rtol=1e-9, atol=1e-10)


def test_mixed_batch_equals_separate_requests():
    lens, news = [90, 200, 64, 33], [1, 70, 4, 33]
    d = synth.decode_inputs(lens, news, 4, 1, 16, 32, kv_dtype=synth.KV_FP8_E4M3FN, seed=33,
                            window=50, with_gate=True, spare_pages=1)
    o, lse = oracle.prefill_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                  d.scale, True, d.k_scale, d.v_scale, window=50, g_cache=d.g_cache)
    cu = d.cu_seqlens_q.numpy()
    for r in range(4):
        a, b = int(cu[r]), int(cu[r + 1])
        o1, l1 = oracle.prefill_paged(d.q[a:b], np.array([0, b - a]), d.k_cache, d.v_cache,
                                      d.block_table[r:r + 1], d.seq_lens[r:r + 1], d.scale, True,
                                      d.k_scale, d.v_scale, window=50, g_cache=d.g_cache)
        np.testing.assert_array_equal(o[a:b], o1)
        np.testing.assert_array_equal(lse[a:b], l1)


@pytest.mark.parametrize("split_len", [32, 64, 128])
def test_split_invariance_for_long_chunks(split_len):
    lens, news = [260, 100], [200, 3]
    d = synth.decode_inputs(lens, news, 4, 1, 16, 16, kv_dtype=synth.KV_FP8_E4M3FN, seed=34,
                            with_sink=True, spare_pages=1)
    o, lse = oracle.prefill_paged(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                  d.scale, True, d.k_scale, d.v_scale, sink=d.sink)
    S = (max(lens) + split_len - 1) // split_len
    acc, m, l = oracle.decode_partials(d.q, d.cu_seqlens_q, d.k_cache, d.v_cache, d.block_table,
                                       d.seq_lens, d.scale, True, split_len, S, d.k_scale, d.v_scale,
                                       sink=d.sink)
    # segments past a row's own position hold empty partials (m = -inf)
    cu = d.cu_seqlens_q.numpy()
    for r, (L, n) in enumerate(zip(lens, news)):
        for t in range(n):
            p = L - n + t
            rows = (cu[r] + t) * 4 + np.arange(4)
            assert np.all(m[rows, p // split_len + 1:] == -np.inf)
    ro, rl = oracle.splitk_reduce(acc, m, l)
    np.testing.assert_allclose(ro.reshape(o.shape), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(rl.reshape(lse.shape), lse, rtol=1e-11, atol=1e-12)
