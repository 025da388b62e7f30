"""Float64 CPU oracle for packed variable-length causal softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark call
it.  It shares no code with the HIP library.

What it computes is the plain materialised definition, written from the fla
issue #1322 "Gluon attention backend with large head dimensions":

  * Description: causal attention over dense or packed variable-length
    inputs, MHA/GQA/MQA, unequal q/k and v head dims, logarithmic gates,
    sliding windows and a sink bias, and their gradients.
  * Comment of Oct 3: the sink gradient is the negative sink probability times
    sum_j P_ij * (dO_i . v_j), reduced over queries.
  * Comment of Oct 5: gate and sink partials are plain sums of the score
    gradient; dQ is the score gradient times K.

Readings taken where the page is silent (each also listed in the design
notes): the gate bias is G_i - G_j with G the inclusive per-sequence cumsum of
g, added after the softmax scale and not multiplied by it; the sink is a raw
per-query-head logit with zero value; a key j is visible from query i iff
j <= i and i - j < window (window <= 0: no window); query head h reads KV head
h // (Hq / Hkv); lse is the natural log of the softmax denominator, sink mass
included.

Everything is float64 on inputs upcast exactly from bf16.  Rows are processed
in blocks only to bound memory; there is no online softmax, tiling or fusion.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):           # torch tensor -> exact float64 copy
        x = x.detach().to("cpu")
        if x.dtype.is_floating_point:
            x = x.double()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.int64)


def gate_prefix(g, cu_seqlens):
    """G[t, h] = sum of g[s, h] over s from the start of t's sequence to t,
    inclusive (the logarithmic gate of the Description; the bias between
    query i and key j is then the sum of g over (j, i])."""
    g = _f64(g)
    cu = _i64(cu_seqlens)
    G = np.zeros_like(g)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        G[a:b] = np.cumsum(g[a:b], axis=0)
    return G


def visible_mask(rows, cols, window):
    """Boolean [len(rows), len(cols)] mask: key j visible from query i iff
    j <= i and (window <= 0 or i - j < window)."""
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) < window
    return m


def _row_block(q_h, K, V, rows, G_h, sink_h, scale, window):
    """Scores, probabilities and statistics for local query rows ``rows`` of
    one sequence and one query head.  Returns (cols, P, psink, m, l) where
    P is [len(rows), len(cols)] over the key columns that can be visible."""
    r0, r1 = rows[0], rows[-1] + 1
    c0 = 0 if window <= 0 else max(0, r0 - window + 1)
    cols = np.arange(c0, r1)
    s = scale * (q_h[r0:r1] @ K[c0:r1].T)
    if G_h is not None:
        s = s + (G_h[r0:r1, None] - G_h[None, c0:r1])
    vis = visible_mask(rows, cols, window)
    s = np.where(vis, s, NEG_INF)
    m = np.max(s, axis=1)
    m = np.maximum(m, sink_h)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    esink = np.exp(sink_h - m) if np.isfinite(sink_h) else np.zeros_like(m)
    l = esink + e.sum(axis=1)
    P = e / l[:, None]
    psink = esink / l
    return cols, P, psink, m, l


def forward(q, k, v, cu_seqlens, scale, window=0, sink=None, g=None,
            row_block=512):
    """o_i = sum_j P_ij v_j and lse_i = m_i + ln(l_i) for every packed token
    and query head.

    q [T, Hq, d_qk], k [T, Hkv, d_qk], v [T, Hkv, d_v], cu_seqlens [N+1],
    sink [Hq] or None, g [T, Hq] or None.  Returns (o [T, Hq, d_v],
    lse [T, Hq]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _i64(cu_seqlens)
    sink = _f64(sink)
    G = gate_prefix(g, cu) if g is not None else None
    T, Hq, _ = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    grp = Hq // Hkv
    o = np.zeros((T, Hq, dv))
    lse = np.zeros((T, Hq))
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        L = b - a
        for h in range(Hq):
            kv = h // grp
            K, V = k[a:b, kv], v[a:b, kv]
            qh = q[a:b, h]
            Gh = None if G is None else G[a:b, h]
            sh = NEG_INF if sink is None else sink[h]
            for r0 in range(0, L, row_block):
                rows = np.arange(r0, min(L, r0 + row_block))
                cols, P, _, m, l = _row_block(qh, K, V, rows, Gh, sh, scale, window)
                o[a + rows, h] = P @ V[cols]
                lse[a + rows, h] = m + np.log(l)
    return o, lse


def backward(q, k, v, do, cu_seqlens, scale, window=0, sink=None, g=None,
             row_block=512, kv_heads=None):
    """Gradients of sum(o * dO) with respect to q, k, v, sink and g.

    With dP_ij = dO_i . v_j and D_i = sum_j P_ij dP_ij (equal to dO_i . o_i,
    computed here without any rounded output):
      dS_ij  = P_ij (dP_ij - D_i)
      dq_i   = scale * sum_j dS_ij k_j
      dk_j   = scale * sum over the group's heads and i of dS_ij q_i
      dv_j   = sum over the group's heads and i of P_ij dO_i
      dsink  = -sum_i psink_i D_i            (Oct 3 comment)
      dG_i   = sum_j dS_ij - sum_i' dS_i'i   (gate bias G_i - G_j)
      dg_t   = sum over i >= t in t's sequence of dG_i
    Returns float64 (dq, dk, dv, dsink or None, dg or None).  With
    ``kv_heads`` given, only those KV heads and their query heads are
    computed (the rest stay zero), for sampled checks of large inputs.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cu = _i64(cu_seqlens)
    sink = _f64(sink)
    G = gate_prefix(g, cu) if g is not None else None
    T, Hq, dqk = q.shape
    Hkv, dvd = k.shape[1], v.shape[2]
    grp = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(Hq) if sink is not None else None
    dG = np.zeros((T, Hq))
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        L = b - a
        for h in range(Hq):
            kv = h // grp
            if kv_heads is not None and kv not in kv_heads:
                continue
            K, V = k[a:b, kv], v[a:b, kv]
            qh, doh = q[a:b, h], do[a:b, h]
            Gh = None if G is None else G[a:b, h]
            sh = NEG_INF if sink is None else sink[h]
            for r0 in range(0, L, row_block):
                rows = np.arange(r0, min(L, r0 + row_block))
                cols, P, psink, _, _ = _row_block(qh, K, V, rows, Gh, sh, scale, window)
                dP = doh[rows] @ V[cols].T
                D = np.sum(P * dP, axis=1)
                dS = P * (dP - D[:, None])
                dq[a + rows, h] = scale * (dS @ K[cols])
                dk[a + cols, kv] += scale * (dS.T @ qh[rows])
                dv[a + cols, kv] += P.T @ doh[rows]
                if dsink is not None:
                    dsink[h] -= np.sum(psink * D)
                dG[a + rows, h] += dS.sum(axis=1)
                dG[a + cols, h] -= dS.sum(axis=0)
    dg = None
    if g is not None:
        dg = np.zeros((T, Hq))
        for n in range(len(cu) - 1):
            a, b = cu[n], cu[n + 1]
            dg[a:b] = np.cumsum(dG[a:b][::-1], axis=0)[::-1]
    return dq, dk, dv, dsink, dg


def row_stats(q, k, cu_seqlens, scale, window=0, sink=None, g=None, heads=None,
              row_block=512):
    """(P-row statistics only) lse [T, Hq] for the listed query heads, NaN
    elsewhere; the cheap half of the forward used when only sampled outputs
    are checked."""
    q, k = _f64(q), _f64(k)
    cu = _i64(cu_seqlens)
    sink = _f64(sink)
    G = gate_prefix(g, cu) if g is not None else None
    T, Hq, _ = q.shape
    grp = Hq // k.shape[1]
    heads = range(Hq) if heads is None else heads
    lse = np.full((T, Hq), np.nan)
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in heads:
            K = k[a:b, h // grp]
            Gh = None if G is None else G[a:b, h]
            sh = NEG_INF if sink is None else sink[h]
            for r0 in range(0, b - a, row_block):
                rows = np.arange(r0, min(b - a, r0 + row_block))
                _, _, _, m, l = _row_block(q[a:b, h], K, None, rows, Gh, sh, scale, window)
                lse[a + rows, h] = m + np.log(l)
    return lse


def forward_rows(q, k, v, cu_seqlens, scale, tokens, heads, window=0, sink=None,
                 g=None):
    """Outputs o[t, h] and lse[t, h] for selected (token, head) pairs only,
    each row computed on its own from the definition.  Returns arrays shaped
    [len(tokens), len(heads), d_v] and [len(tokens), len(heads)]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _i64(cu_seqlens)
    sink = _f64(sink)
    g = _f64(g)
    Hq, Hkv = q.shape[1], k.shape[1]
    grp = Hq // Hkv
    out = np.zeros((len(tokens), len(heads), v.shape[2]))
    lse = np.zeros((len(tokens), len(heads)))
    for ti, t in enumerate(tokens):
        n = int(np.searchsorted(cu, t, side="right") - 1)
        a = cu[n]
        i = t - a
        for hi, h in enumerate(heads):
            kv = h // grp
            j0 = 0 if window <= 0 else max(0, i - window + 1)
            js = np.arange(j0, i + 1)
            s = scale * (k[a + js, kv] @ q[t, h])
            if g is not None:
                Gi = np.sum(g[a:a + i + 1, h])
                Gj = np.cumsum(g[a:a + i + 1, h])[js]
                s = s + (Gi - Gj)
            sh = NEG_INF if sink is None else sink[h]
            m = max(np.max(s), sh)
            e = np.exp(s - m)
            l = e.sum() + (np.exp(sh - m) if np.isfinite(sh) else 0.0)
            out[ti, hi] = (e / l) @ v[a + js, kv]
            lse[ti, hi] = m + np.log(l)
    return out, lse
