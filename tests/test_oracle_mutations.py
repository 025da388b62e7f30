"""Planted mistakes in (copies of) the oracle must fail its pins.

Each test swaps one oracle helper for a plausibly wrong variant (on the CPU
only, restored afterwards) and checks that the independent pin it is meant to
be caught by does reject it.  This shows that the pins constrain the pieces
they are meant to constrain.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od
from oracle import prefill as op
from tests.test_oracle_prefill import _case, _torch_ref


def _forward_mismatch(window=4, sink=True, gate=True, heads=(4, 2)):
    q, k, v, do, cu, s, g = _case([6, 11], heads[0], heads[1], 8, 8, seed=41,
                                  sink=sink, gate=gate)
    o, _ = op.forward(q, k, v, cu, 0.5, window, s, g)
    ro, _, _ = _torch_ref(q, k, v, cu, 0.5, window, s, g)
    return np.max(np.abs(o - ro))


def test_pins_accept_unmutated():
    assert _forward_mismatch() < 1e-12


def test_window_off_by_one_is_caught(monkeypatch):
    def wrong(rows, cols, window):
        i = np.asarray(rows)[:, None]; j = np.asarray(cols)[None, :]
        m = j <= i
        if window > 0:
            m &= (i - j) <= window
        return m
    monkeypatch.setattr(op, "visible_mask", wrong)
    assert _forward_mismatch() > 1e-3


def test_gate_sign_flip_is_caught(monkeypatch):
    right = op.gate_prefix
    monkeypatch.setattr(op, "gate_prefix", lambda g, cu: -right(g, cu))
    assert _forward_mismatch() > 1e-3


def test_exclusive_cumsum_is_caught(monkeypatch):
    right = op.gate_prefix
    monkeypatch.setattr(op, "gate_prefix",
                        lambda g, cu: right(g, cu) - np.asarray(g, dtype=np.float64))
    assert _forward_mismatch() > 1e-3


def test_dropped_sink_is_caught(monkeypatch):
    right = op._row_block
    monkeypatch.setattr(op, "_row_block",
                        lambda qh, K, V, rows, G, sh, sc, w: right(qh, K, V, rows, G, -np.inf, sc, w))
    assert _forward_mismatch() > 1e-3


def test_wrong_gqa_mapping_is_caught():
    # an oracle that pairs query head h with KV head h % Hkv instead of
    # h // (Hq / Hkv): emulate by permuting heads of K/V for the oracle only
    q, k, v, do, cu, s, g = _case([9], 4, 2, 8, 8, seed=42)
    o_wrong, _ = op.forward(q, k[:, ::-1].copy(), v[:, ::-1].copy(), cu, 0.5, 0, s, g)
    ro, _, _ = _torch_ref(q, k, v, cu, 0.5, 0, s, g)
    assert np.max(np.abs(o_wrong - ro)) > 1e-3


def test_fp8_wrong_bias_is_caught(monkeypatch):
    # an oracle whose e4m3fn decoder uses exponent bias 8 instead of 7 must
    # fail both fp8 pins (all 256 codes against torch, and the format's
    # fixed points)
    from tests import test_oracle_decode as pins

    def wrong(codes):
        c = np.asarray(codes).astype(np.int64)
        s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
        sign = np.where(s == 1, -1.0, 1.0)
        out = np.where(e == 0, sign * (m / 8.0) * 2.0 ** -7,
                       sign * (1.0 + m / 8.0) * np.power(2.0, (e - 8).astype(np.float64)))
        return np.where((e == 15) & (m == 7), np.nan, out)

    monkeypatch.setattr(oracle, "fp8_e4m3fn_to_f64", wrong)
    monkeypatch.setattr(od, "fp8_e4m3fn_to_f64", wrong)
    with pytest.raises(AssertionError):
        pins.test_fp8_decode_matches_torch_on_all_codes()
    with pytest.raises(AssertionError):
        pins.test_fp8_format_fixed_points()


def test_sink_gradient_sign_flip_is_caught():
    q, k, v, do, cu, s, g = _case([7], 2, 1, 4, 4, seed=43)
    _, _, rg = _torch_ref(q, k, v, cu, 0.5, 0, s, g, do)
    ds = op.backward(q, k, v, do, cu, 0.5, 0, s, g)[3]
    assert np.allclose(ds, rg[3], rtol=1e-10)
    assert not np.allclose(-ds, rg[3], rtol=1e-3)


def test_reduce_without_rescale_is_caught():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(30) * 4
    V = rng.standard_normal((30, 2))
    acc = np.zeros((1, 2, 2)); m = np.zeros((1, 2)); l = np.zeros((1, 2))
    for s, (a, b) in enumerate([(0, 11), (11, 30)]):
        m[0, s] = x[a:b].max(); e = np.exp(x[a:b] - m[0, s])
        l[0, s] = e.sum(); acc[0, s] = e @ V[a:b]
    p = np.exp(x - x.max()); p /= p.sum()
    o, _ = od.splitk_reduce(acc, m, l)
    assert np.allclose(o[0], p @ V, rtol=1e-12)
    wrong = acc[0].sum(0) / l[0].sum()                 # forgot exp(m_s - M)
    assert not np.allclose(wrong, p @ V, rtol=1e-3)
