"""Pins for the prefill oracle against things other than itself.

  * torch float64 scaled_dot_product_attention (math path) with an explicit
    extra sink key (k = 0, v = 0, mask entry = sink logit) and a float mask
    carrying G_i - G_j -- an independent library implementation;
  * torch autograd through that graph for dq, dk, dv, dsink and dg;
  * central finite differences of sum(o * dO) through the oracle forward;
  * closed forms (one-token sequences; q = 0 gives uniform attention);
  * invariants (rows of P plus the sink mass sum to 1, dsink = -sum dS,
    dg at each sequence start is 0, GQA = MHA with repeated K/V, packing
    = separate runs, window edge counts);
  * brute force with scalar Python loops on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill as op
from tests.util import rel_rms


def _case(seqlens, Hq, Hkv, dqk, dv, seed, sink=True, gate=True):
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    q = rng.standard_normal((T, Hq, dqk))
    k = rng.standard_normal((T, Hkv, dqk))
    v = rng.standard_normal((T, Hkv, dv))
    do = rng.standard_normal((T, Hq, dv))
    s = rng.standard_normal(Hq) if sink else None
    g = np.log(1.0 / (1.0 + np.exp(-(rng.standard_normal((T, Hq)) + 3.0)))) if gate else None
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return q, k, v, do, cu, s, g


def _torch_ref(q, k, v, cu, scale, window, sink, g, do=None):
    """Library reference: per sequence, SDPA over K/V with one extra key of
    zeros whose mask entry is the sink logit."""
    Hq, Hkv = q.shape[1], k.shape[1]
    grp = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    ts = torch.tensor(sink, requires_grad=True) if sink is not None else None
    tg = torch.tensor(g, requires_grad=True) if g is not None else None
    outs, lses = [], []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        L = b - a
        qn = tq[a:b].transpose(0, 1)                                  # [Hq,L,d]
        kn = tk[a:b].repeat_interleave(grp, dim=1).transpose(0, 1)     # [Hq,L,d]
        vn = tv[a:b].repeat_interleave(grp, dim=1).transpose(0, 1)
        kx = torch.cat([kn, torch.zeros(Hq, 1, kn.shape[2], dtype=kn.dtype)], 1)
        vx = torch.cat([vn, torch.zeros(Hq, 1, vn.shape[2], dtype=vn.dtype)], 1)
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        vis = j <= i
        if window > 0:
            vis = vis & (i - j < window)
        bias = torch.zeros(Hq, L, L, dtype=torch.float64)
        if tg is not None:
            G = torch.cumsum(tg[a:b], dim=0).transpose(0, 1)          # [Hq, L]
            bias = G[:, :, None] - G[:, None, :]
        bias = torch.where(vis[None], bias, torch.full_like(bias, -math.inf))
        sc = ts[:, None, None].expand(Hq, L, 1) if ts is not None else \
            torch.full((Hq, L, 1), -math.inf, dtype=torch.float64)
        mask = torch.cat([bias, sc], dim=2)
        o = torch.nn.functional.scaled_dot_product_attention(
            qn[None], kx[None], vx[None], attn_mask=mask[None], scale=scale)[0]
        logits = scale * (qn @ kx.transpose(1, 2)) + mask
        lses.append(torch.logsumexp(logits, dim=2).transpose(0, 1))
        outs.append(o.transpose(0, 1))
    O = torch.cat(outs, 0)
    LSE = torch.cat(lses, 0)
    grads = None
    if do is not None:
        (O * torch.tensor(do)).sum().backward()
        grads = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(),
                 None if ts is None else ts.grad.numpy(),
                 None if tg is None else tg.grad.numpy())
    return O.detach().numpy(), LSE.detach().numpy(), grads


FEATURES = [
    dict(sink=False, gate=False, window=0),
    dict(sink=True, gate=False, window=0),
    dict(sink=False, gate=True, window=0),
    dict(sink=False, gate=False, window=4),
    dict(sink=True, gate=True, window=5),
]


@pytest.mark.parametrize("feat", FEATURES, ids=lambda f: "-".join(
    k for k, v in f.items() if v))
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (6, 1)], ids=["mha", "gqa2", "mqa"])
def test_forward_backward_match_torch_library(feat, heads):
    Hq, Hkv = heads
    q, k, v, do, cu, s, g = _case([5, 17, 1, 23], Hq, Hkv, 8, 12, seed=11,
                                  sink=feat["sink"], gate=feat["gate"])
    scale = 0.37
    o, lse = oracle.forward(q, k, v, cu, scale, feat["window"], s, g, row_block=7)
    ro, rlse, rg = _torch_ref(q, k, v, cu, scale, feat["window"], s, g, do)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-12, atol=1e-12)
    dq, dk, dv, ds, dg = oracle.backward(q, k, v, do, cu, scale, feat["window"], s, g,
                                         row_block=6)
    np.testing.assert_allclose(dq, rg[0], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, rg[1], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, rg[2], rtol=1e-10, atol=1e-11)
    if s is not None:
        np.testing.assert_allclose(ds, rg[3], rtol=1e-10, atol=1e-11)
    else:
        assert ds is None
    if g is not None:
        np.testing.assert_allclose(dg, rg[4], rtol=1e-10, atol=1e-10)
    else:
        assert dg is None


def test_plain_causal_reduces_to_is_causal():
    q, k, v, do, cu, _, _ = _case([19], 3, 3, 16, 16, seed=3, sink=False, gate=False)
    o, _ = oracle.forward(q, k, v, cu, 0.25, 0, None, None)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
        torch.tensor(v).transpose(0, 1), is_causal=True, scale=0.25).transpose(0, 1)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def _loss(q, k, v, do, cu, scale, window, s, g):
    o, _ = oracle.forward(q, k, v, cu, scale, window, s, g)
    return float(np.sum(o * do))


def test_gradients_match_finite_differences():
    """Central differences (h = 1e-6, float64) of sum(o * dO) on two packed
    sequences of 3 and 5 tokens, Hq 2 / Hkv 1, d_qk 4, d_v 3, window 3, with
    sink and gates, for every input including the sink and the gates."""
    q, k, v, do, cu, s, g = _case([3, 5], 2, 1, 4, 3, seed=5)
    scale, W, h = 0.6, 3, 1e-6
    grads = oracle.backward(q, k, v, do, cu, scale, W, s, g)
    args = dict(q=q, k=k, v=v, s=s, g=g)
    for gi, name in enumerate(["q", "k", "v", "s", "g"]):
        x = args[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = dict(args, **{name: xp})
            am = dict(args, **{name: xm})
            fp = _loss(ap["q"], ap["k"], ap["v"], do, cu, scale, W, ap["s"], ap["g"])
            fm = _loss(am["q"], am["k"], am["v"], do, cu, scale, W, am["s"], am["g"])
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(grads[gi], num, rtol=1e-6, atol=1e-8,
                                   err_msg=f"d{name}")


def test_single_token_closed_form():
    """L = 1: o_0 = v_0 / (1 + exp(sink - scale q.k)); lse = log(e^s + e^sink)."""
    q, k, v, do, cu, s, g = _case([1, 1, 1], 2, 1, 8, 5, seed=9)
    scale = 0.3
    o, lse = oracle.forward(q, k, v, cu, scale, 0, s, g)
    for t in range(3):
        for h in range(2):
            s00 = scale * q[t, h] @ k[t, 0]
            np.testing.assert_allclose(o[t, h], v[t, 0] / (1 + np.exp(s[h] - s00)),
                                       rtol=1e-13)
            np.testing.assert_allclose(lse[t, h], np.logaddexp(s00, s[h]), rtol=1e-13)


def test_zero_query_uniform_closed_form():
    """q = 0 and g = 0, no window: P_ij = 1 / (i + 1 + e^sink), so
    o_i = sum_{j<=i} v_j / (i + 1 + e^sink)."""
    q, k, v, do, cu, s, _ = _case([9], 3, 1, 4, 6, seed=2, gate=False)
    q[:] = 0.0
    o, lse = oracle.forward(q, k, v, cu, 1.0, 0, s, None)
    for i in range(9):
        for h in range(3):
            den = i + 1 + np.exp(s[h])
            np.testing.assert_allclose(o[i, h], v[:i + 1, 0].sum(0) / den, rtol=1e-13)
            np.testing.assert_allclose(lse[i, h], np.log(den), rtol=1e-13)


def test_probabilities_plus_sink_sum_to_one():
    q, k, v, do, cu, s, g = _case([13], 2, 1, 8, 8, seed=4)
    G = oracle.gate_prefix(g, cu)
    for h in range(2):
        cols, P, psink, m, l = op._row_block(q[:, h], k[:, 0], v[:, 0],
                                             np.arange(13), G[:, h], s[h], 0.5, 6)
        np.testing.assert_allclose(P.sum(1) + psink, 1.0, rtol=0, atol=1e-14)
        assert np.all(P >= 0) and np.all(psink > 0)
        # exactly min(i + 1, W) visible keys per row
        np.testing.assert_array_equal((P > 0).sum(1), np.minimum(np.arange(13) + 1, 6))


def test_sink_gradient_equals_minus_sum_of_score_gradient():
    """sum_j dS_ij = D_i psink_i, so dsink_h = -sum over i, j of dS_ij."""
    q, k, v, do, cu, s, g = _case([7, 11], 4, 2, 8, 8, seed=6)
    scale, W = 0.4, 5
    _, _, _, ds, _ = oracle.backward(q, k, v, do, cu, scale, W, s, g)
    G = oracle.gate_prefix(g, cu)
    tot = np.zeros(4)
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        for h in range(4):
            cols, P, psink, _, _ = op._row_block(q[a:b, h], k[a:b, h // 2], v[a:b, h // 2],
                                                 np.arange(b - a), G[a:b, h], s[h], scale, W)
            dP = do[a:b, h] @ v[a:b, h // 2][cols].T
            D = (P * dP).sum(1)
            tot[h] -= (P * (dP - D[:, None])).sum()
    np.testing.assert_allclose(ds, tot, rtol=1e-11)


def test_gate_gradient_vanishes_at_sequence_start():
    """dg_start = sum_i dG_i = 0: the bias G_i - G_j does not change when a
    constant is added to every G of a sequence."""
    q, k, v, do, cu, s, g = _case([6, 10, 4], 2, 2, 8, 8, seed=8)
    _, _, _, _, dg = oracle.backward(q, k, v, do, cu, 0.5, 4, s, g)
    assert np.max(np.abs(dg[cu[:-1]])) < 1e-12
    assert np.max(np.abs(dg)) > 1e-3


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v, do, cu, s, g = _case([8, 9], 6, 2, 8, 4, seed=12)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o1, l1 = oracle.forward(q, k, v, cu, 0.3, 3, s, g)
    o2, l2 = oracle.forward(q, kr, vr, cu, 0.3, 3, s, g)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    b1 = oracle.backward(q, k, v, do, cu, 0.3, 3, s, g)
    b2 = oracle.backward(q, kr, vr, do, cu, 0.3, 3, s, g)
    np.testing.assert_allclose(b1[0], b2[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b1[1], b2[1].reshape(17, 2, 3, 8).sum(2), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b1[2], b2[2].reshape(17, 2, 3, 4).sum(2), rtol=1e-12, atol=1e-14)


def test_packed_equals_separate_sequences():
    q, k, v, do, cu, s, g = _case([4, 12, 7], 2, 1, 8, 8, seed=13)
    o, lse = oracle.forward(q, k, v, cu, 0.5, 5, s, g, row_block=3)
    grads = oracle.backward(q, k, v, do, cu, 0.5, 5, s, g, row_block=3)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        c1 = np.array([0, b - a])
        o1, l1 = oracle.forward(q[a:b], k[a:b], v[a:b], c1, 0.5, 5, s, g[a:b])
        np.testing.assert_allclose(o[a:b], o1, rtol=1e-14, atol=1e-15)
        g1 = oracle.backward(q[a:b], k[a:b], v[a:b], do[a:b], c1, 0.5, 5, s, g[a:b])
        for x, y in zip(grads[:3], g1[:3]):
            np.testing.assert_allclose(x[a:b], y, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(grads[4][a:b], g1[4], rtol=1e-12, atol=1e-14)


def test_window_edge():
    """With W = 3, query i sees keys i-2..i: moving a key from distance 2 to
    distance 3 (by making only one visible key carry a large value) shows
    the edge.  Keys at distance W-1 are visible, at W and W+1 not."""
    L, W = 8, 3
    q = np.zeros((L, 1, 1)); k = np.zeros((L, 1, 1))
    for dist in (W - 1, W, W + 1):
        v = np.zeros((L, 1, 1))
        v[L - 1 - dist, 0, 0] = 1.0
        o, _ = oracle.forward(q, k, v, np.array([0, L]), 1.0, W, None, None)
        expect = 1.0 / W if dist < W else 0.0
        assert abs(o[L - 1, 0, 0] - expect) < 1e-15, dist


def _brute_forward(q, k, v, cu, scale, W, s, g):
    T, Hq, _ = q.shape
    grp = Hq // k.shape[1]
    o = np.zeros((T, Hq, v.shape[2]))
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in range(Hq):
            for i in range(b - a):
                logits = []
                for j in range(b - a):
                    if j > i or (W > 0 and i - j >= W):
                        continue
                    x = scale * sum(q[a + i, h, d] * k[a + j, h // grp, d]
                                    for d in range(q.shape[2]))
                    if g is not None:
                        x += sum(g[a + t, h] for t in range(j + 1, i + 1))
                    logits.append((j, x))
                mx = max([x for _, x in logits] + ([s[h]] if s is not None else []))
                den = sum(math.exp(x - mx) for _, x in logits)
                if s is not None:
                    den += math.exp(s[h] - mx)
                for j, x in logits:
                    o[a + i, h] += math.exp(x - mx) / den * v[a + j, h // grp]
    return o


def test_brute_force_loops():
    q, k, v, do, cu, s, g = _case([3, 6, 1], 4, 2, 3, 2, seed=21)
    for W in (0, 2):
        o, _ = oracle.forward(q, k, v, cu, 0.7, W, s, g)
        np.testing.assert_allclose(o, _brute_forward(q, k, v, cu, 0.7, W, s, g),
                                   rtol=1e-12, atol=1e-14)


def test_forward_rows_and_row_stats_agree_with_full():
    q, k, v, do, cu, s, g = _case([20, 33], 4, 2, 8, 6, seed=31)
    o, lse = oracle.forward(q, k, v, cu, 0.5, 7, s, g)
    toks = [0, 5, 19, 20, 21, 52]
    heads = [0, 3]
    ro, rl = oracle.forward_rows(q, k, v, cu, 0.5, toks, heads, 7, s, g)
    np.testing.assert_allclose(ro, o[np.ix_(toks, heads)], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rl, lse[np.ix_(toks, heads)], rtol=1e-12)
    st = oracle.row_stats(q, k, cu, 0.5, 7, s, g, heads=[1, 2])
    np.testing.assert_allclose(st[:, 1:3], lse[:, 1:3], rtol=1e-12)
    assert np.isnan(st[:, 0]).all()


def test_backward_kv_head_subset():
    q, k, v, do, cu, s, g = _case([10, 7], 4, 2, 8, 6, seed=32)
    full = oracle.backward(q, k, v, do, cu, 0.5, 0, s, g)
    sub = oracle.backward(q, k, v, do, cu, 0.5, 0, s, g, kv_heads=[1])
    np.testing.assert_allclose(sub[0][:, 2:], full[0][:, 2:], rtol=1e-13)
    np.testing.assert_allclose(sub[1][:, 1], full[1][:, 1], rtol=1e-13)
    np.testing.assert_allclose(sub[2][:, 1], full[2][:, 1], rtol=1e-13)
    np.testing.assert_allclose(sub[3][2:], full[3][2:], rtol=1e-13)
    np.testing.assert_allclose(sub[4][:, 2:], full[4][:, 2:], rtol=1e-13, atol=1e-15)
