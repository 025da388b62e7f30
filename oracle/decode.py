"""Float64 CPU oracle for paged decode, split-K partials and their LSE merge.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark call
it.  It shares no code with the HIP library.

Written from ROCm/aiter PR #6660 ("per-token fp8 KV scales and short-query
split-K"):
  * commit message 1 and "Technical details": one float32 K and one V scale
    per cached token and KV head, laid out [num_blocks, num_kv_heads,
    block_size]; each score column is scaled by its key's K scale, each
    probability column by its key's V scale once the row sum has been taken;
    slots past seq_len contribute nothing;
  * commit message 2: the scaled probabilities must meet V at fp32 accuracy
    (here: exactly, in float64);
  * commit message 3 and "Technical details": queries of a few tokens per
    request over long contexts, split into KV segments whose partials are
    merged by a log-sum-exp reduce; a query whose visible keys end before a
    segment gives an empty partial (M = -inf) of weight 0.

Decode features of the prefill method (fla issue #1322, Description: the
packed single-query decoding counterparts of the sink, sliding window and
log gate), with the same definitions as the prefill oracle: a per-query-head
sink logit adds e^sigma to the denominator; key j is visible from the query
at position p iff p - j < window (window <= 0: no window); the score gains
G_p - G_j with G the cumulative log gate of each token and query head, read
from a paged gate cache [num_blocks, Hq, block_size] at the key's and at the
query's own position.  Per-tensor scales (one K and one V scale for the whole
cache) replace the per-token ones when ``per_tensor`` is set.

Readings: the cache data layout is [num_blocks, num_kv_heads, block_size, D];
token j of request r sits in page block_table[r][j // B], slot j % B; query t
of a request with KV length L and n new tokens sits at position L - n + t and
sees keys 0..L-n+t; fp8 is OCP e4m3fn; a partial is (unnormalised acc, m, l)
with natural-log m.
"""
from __future__ import annotations

import numpy as np

from .prefill import _f64, _i64

NEG_INF = -np.inf


def fp8_e4m3fn_to_f64(codes):
    """Decode OCP e4m3fn bytes s.eeee.mmm (exponent bias 7, no infinities):
    e = 15 and m = 7 is NaN; e = 0 is subnormal (-1)^s (m/8) 2^-6; otherwise
    (-1)^s (1 + m/8) 2^(e-7).  Largest finite magnitude 448."""
    c = _i64(codes)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    nrm = sign * (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    out = np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, out)


def gather_request_kv(cache, scale, block_table, r, L, B, fp8, per_tensor=False):
    """Dequantised keys (or values) of request r: [L, Hkv, D] float64, token
    j read from page block_table[r][j // B], slot j % B, times its per-token
    scale for fp8 (or the single per-tensor scale)."""
    bt = _i64(block_table)
    j = np.arange(L)
    pages = bt[r, j // B]
    slots = j % B
    raw = cache[pages, :, slots, :]            # [L, Hkv, D]
    if fp8:
        x = fp8_e4m3fn_to_f64(raw)
        if per_tensor:
            return x * float(np.asarray(_f64(scale)).reshape(-1)[0])
        sc = _f64(scale)[pages, :, slots]      # [L, Hkv]
        return x * sc[..., None]
    return _f64(raw)


def gather_request_gates(g_cache, block_table, r, L, B):
    """Cumulative log gates of request r's tokens: [L, Hq] float64, token j
    read from page block_table[r][j // B], slot j % B of g_cache
    [num_blocks, Hq, B]."""
    bt = _i64(block_table)
    j = np.arange(L)
    return _f64(g_cache)[bt[r, j // B], :, j % B]


def _as_cache(c):
    if hasattr(c, "detach"):
        c = c.detach().to("cpu")
        import torch  # only to read bf16 storage exactly
        if c.dtype == torch.bfloat16:
            return c.double().numpy()
        return c.numpy()
    return np.asarray(c)


def decode_paged(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens,
                 scale, fp8, k_scale=None, v_scale=None, requests=None,
                 sink=None, window=0, g_cache=None, per_tensor=False):
    """o[t, h] = softmax over the visible keys of
    s_j = scale * q_t . Khat_j + (G_p - G_j) (gate term only with a gate
    cache), with e^sink[h] added to the denominator when a sink is given;
    visible keys are j <= p with p - j < window (window <= 0: all j <= p).
    Also lse[t, h] (natural log, sink mass included).

    Returns (o [Tq, Hq, D], lse [Tq, Hq]) float64.  With ``requests`` given,
    only those requests' rows are filled (others NaN).
    """
    q = _f64(q)
    cu = _i64(cu_seqlens_q)
    L_all = _i64(seq_lens)
    kc, vc = _as_cache(k_cache), _as_cache(v_cache)
    sink = None if sink is None else _f64(sink)
    B = kc.shape[2]
    Tq, Hq, D = q.shape
    Hkv = kc.shape[1]
    grp = Hq // Hkv
    o = np.full((Tq, Hq, vc.shape[3]), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    reqs = range(len(cu) - 1) if requests is None else requests
    for r in reqs:
        L = int(L_all[r])
        n = int(cu[r + 1] - cu[r])
        K = gather_request_kv(kc, k_scale, block_table, r, L, B, fp8, per_tensor)
        V = gather_request_kv(vc, v_scale, block_table, r, L, B, fp8, per_tensor)
        G = None if g_cache is None else gather_request_gates(g_cache, block_table, r, L, B)
        for t in range(n):
            p = L - n + t
            j0 = 0 if window <= 0 else max(0, p - window + 1)
            for h in range(Hq):
                s = scale * (K[j0:p + 1, h // grp] @ q[cu[r] + t, h])
                if G is not None:
                    s = s + (G[p, h] - G[j0:p + 1, h])
                sh = -np.inf if sink is None else sink[h]
                m = max(np.max(s), sh)
                e = np.exp(s - m)
                l = e.sum() + (np.exp(sh - m) if np.isfinite(sh) else 0.0)
                o[cu[r] + t, h] = (e / l) @ V[j0:p + 1, h // grp]
                lse[cu[r] + t, h] = m + np.log(l)
    return o, lse


def prefill_paged(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens,
                  scale, fp8, k_scale=None, v_scale=None, sink=None, window=0,
                  g_cache=None, per_tensor=False):
    """Paged prefill over the same cache: any number n >= 1 of new tokens per
    request (chunked prefill, speculative verify longer than four tokens, or
    a mixed batch of these with decode rows).

    ROCm/aiter PR #6660, "Technical details" and commit message 3: batches
    that are not all short queries take the other ("2d") kernel, with one
    program per (KV head, query block) over the paged cache.  The per-row
    definition does not depend on the route: query t of a request with KV
    length L and n new tokens sits at position L - n + t and its output is
    the softmax-weighted sum over its visible keys, exactly as in
    ``decode_paged``, which this evaluates row by row.
    """
    return decode_paged(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, scale, fp8,
                        k_scale, v_scale, sink=sink, window=window, g_cache=g_cache,
                        per_tensor=per_tensor)


def decode_partials(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens,
                    scale, fp8, split_len, num_splits, k_scale=None,
                    v_scale=None, sink=None, window=0, g_cache=None,
                    per_tensor=False):
    """Split-K partials over KV segments [s*split_len, (s+1)*split_len) of
    each request, for every query row (row = token * Hq + head):
      m_s   = max of the logits (as in decode_paged) of the segment's keys
              that the query sees, or -inf when it sees none of them;
      l_s   = sum of exp(logit - m_s) over those keys;
      acc_s = sum of exp(logit - m_s) Vhat_j over those keys.
    The sink, when given, belongs to segment 0: m_0 = max(sink, ...) and l_0
    gains exp(sink - m_0) (it carries no value).  Empty partials carry l = 0
    and acc = 0.  Returns (acc [rows, S, D], m [rows, S], l [rows, S])
    float64 with S = num_splits.
    """
    q = _f64(q)
    cu = _i64(cu_seqlens_q)
    L_all = _i64(seq_lens)
    kc, vc = _as_cache(k_cache), _as_cache(v_cache)
    sink = None if sink is None else _f64(sink)
    B = kc.shape[2]
    Tq, Hq, D = q.shape
    Dv = vc.shape[3]
    grp = Hq // kc.shape[1]
    acc = np.zeros((Tq * Hq, num_splits, Dv))
    m = np.full((Tq * Hq, num_splits), NEG_INF)
    l = np.zeros((Tq * Hq, num_splits))
    for r in range(len(cu) - 1):
        L = int(L_all[r])
        n = int(cu[r + 1] - cu[r])
        K = gather_request_kv(kc, k_scale, block_table, r, L, B, fp8, per_tensor)
        V = gather_request_kv(vc, v_scale, block_table, r, L, B, fp8, per_tensor)
        G = None if g_cache is None else gather_request_gates(g_cache, block_table, r, L, B)
        for t in range(n):
            p = L - n + t
            lo = 0 if window <= 0 else max(0, p - window + 1)
            for h in range(Hq):
                row = (cu[r] + t) * Hq + h
                for s_ in range(num_splits):
                    j0 = max(s_ * split_len, lo)
                    j1 = min((s_ + 1) * split_len, p + 1)
                    sh = sink[h] if (sink is not None and s_ == 0) else -np.inf
                    if j1 <= j0 and not np.isfinite(sh):
                        continue
                    if j1 > j0:
                        sc = scale * (K[j0:j1, h // grp] @ q[cu[r] + t, h])
                        if G is not None:
                            sc = sc + (G[p, h] - G[j0:j1, h])
                    else:
                        sc = np.zeros(0)
                    ms = max(np.max(sc) if sc.size else -np.inf, sh)
                    e = np.exp(sc - ms)
                    m[row, s_] = ms
                    l[row, s_] = e.sum() + (np.exp(sh - ms) if np.isfinite(sh) else 0.0)
                    acc[row, s_] = e @ V[j0:j1, h // grp] if sc.size else 0.0
    return acc, m, l


def splitk_reduce(acc, m, l):
    """Merge partials per row: M = max_s m_s; w_s = exp(m_s - M), or 0 when
    m_s = -inf (acc and l of such a split are never read); L = sum_s w_s l_s;
    o = sum_s w_s acc_s / L; lse = M + ln L.  A row whose partials are all
    empty gives o = 0 and lse = -inf.  Returns float64 (o [rows, Dv],
    lse [rows])."""
    acc, m, l = _f64(acc), _f64(m), _f64(l)
    rows, S, Dv = acc.shape
    o = np.zeros((rows, Dv))
    lse = np.full(rows, NEG_INF)
    for r in range(rows):
        live = np.isfinite(m[r])
        if not live.any():
            continue
        M = np.max(m[r][live])
        w = np.exp(m[r][live] - M)
        Lsum = np.sum(w * l[r][live])
        o[r] = (w[:, None] * acc[r][live]).sum(axis=0) / Lsum
        lse[r] = M + np.log(Lsum)
    return o, lse
