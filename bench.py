#!/usr/bin/env python3
"""Benchmark of the causal softmax attention hot path on one MI355X.

One step = one pass over every hot-path step on synthetic inputs already
resident in HBM:
  * prefill: attn_fwd_varlen + attn_bwd_varlen on the packed varlen workload
    (8 sequences of seeded lengths in [256, 4096], 32 query / 8 KV heads,
    head dim 128, window 1024, sink and log gates) -- tile schedule, gate
    prefix, forward tile loop, backward pre / fused / post;
  * decode: attn_decode_paged on 64 requests with contexts in [1, 32768],
    64 query / 4 KV heads, head dim 128, page 16, per-token fp8 KV, one query
    token each -- split-K partials and the LSE reduce (one layer).

Prints ONE JSON line.  `value` is the prefill fwd+bwd throughput in TFLOP/s
(algorithmic flops: visible (query, key) pairs only); the decode figures
(us per layer, GB/s of algorithmic bytes) sit in `decode`.  Every API call is
bracketed by HIP events on the stream it runs on.  `roofline` describes the
call with the largest share of the step; `cpu_baseline` is the float64 CPU
oracle timed on a bounded sample of the same prefill workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12   # 2516.6 dense bf16
HBM_PEAK_GBPS = 8000.0


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "causal_softmax_attention_amd", "csrc")


def kernel_sources_digest():
    """sha256 over the HIP sources (file names and bytes, sorted)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def stored_traffic(call):
    """HBM bytes per call of `call` measured with rocprofv3 counters
    (profiles/hbm_traffic.txt, lines `call sources=<sha256> bytes=<n>`), or
    None when absent or taken on kernel sources other than the current ones."""
    path = os.path.join(PROFILES, "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest()
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) < 3 or line.startswith("#") or parts[0] != call:
                continue
            kv = dict(p.split("=", 1) for p in parts[1:] if "=" in p)
            if kv.get("sources") == digest and "bytes" in kv:
                return float(kv["bytes"])
    return None


def visible_pairs(seqlens, window):
    tot = 0
    for L in seqlens:
        if window > 0 and L > window:
            tot += window * (window + 1) // 2 + (L - window) * window
        else:
            tot += L * (L + 1) // 2
    return tot


def prefill_flops(x):
    Hq, dqk = x.q.shape[1], x.q.shape[2]
    dv = x.v.shape[2]
    pairs = visible_pairs(x.seqlens, x.window)
    return 2 * pairs * Hq * (dqk + dv), 2 * pairs * Hq * (3 * dqk + 2 * dv), pairs


def decode_bytes(d):
    L = d.seq_lens.to(torch.int64).sum().item()
    Hkv, D = d.k_cache.shape[1], d.k_cache.shape[3]
    elem = 1 if d.kv_dtype == 1 else 2
    b = L * Hkv * 2 * D * elem
    if d.kv_dtype == 1:
        b += L * Hkv * 8
    b += d.q.numel() * 2 * 2                       # q in, o out (bf16)
    pages = sum(math.ceil(int(x) / d.block_size) for x in d.seq_lens.tolist())
    b += pages * 4                                 # block-table entries read
    return b


class Timer:
    """HIP events on the current stream around each API call."""

    def __init__(self):
        self.t = {}

    def run(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.t.setdefault(name, []).append((s, e))
        return r

    def mean_us(self, name):
        ev = self.t.get(name, [])
        return 1e3 * sum(s.elapsed_time(e) for s, e in ev) / max(1, len(ev))

    def median_us(self, name):
        ev = self.t.get(name, [])
        return 1e3 * float(np.median([s.elapsed_time(e) for s, e in ev])) if ev else 0.0


def cpu_oracle_baseline(x, budget_s=12.0):
    """The float64 oracle, as it stands, on a bounded sample of the prefill
    workload: whole KV-head groups of the first sequences, until ~budget_s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cu = x.cu_seqlens.cpu().numpy()
    Hq, Hkv = x.q.shape[1], x.k.shape[1]
    grp = Hq // Hkv
    q, k, v, do = (t.cpu() for t in (x.q, x.k, x.v, x.do))
    sink = x.sink.cpu() if x.sink is not None else None
    g = x.g.cpu() if x.g is not None else None
    flops, spent, done = 0, 0.0, []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        c1 = np.array([0, b - a])
        for kv in range(Hkv):
            hs = slice(kv * grp, (kv + 1) * grp)
            t0 = time.perf_counter()
            oracle.forward(q[a:b, hs], k[a:b, kv:kv + 1], v[a:b, kv:kv + 1], c1, x.scale, x.window,
                           None if sink is None else sink[hs], None if g is None else g[a:b, hs])
            oracle.backward(q[a:b, hs], k[a:b, kv:kv + 1], v[a:b, kv:kv + 1], do[a:b, hs], c1,
                            x.scale, x.window, None if sink is None else sink[hs],
                            None if g is None else g[a:b, hs])
            spent += time.perf_counter() - t0
            pairs = visible_pairs([b - a], x.window)
            dqk, dv = x.q.shape[2], x.v.shape[2]
            flops += 2 * pairs * grp * ((dqk + dv) + (3 * dqk + 2 * dv))
            done.append(f"seq{n}(L={b - a})/kv{kv}")
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 oracle forward+backward on {len(done)} (sequence, KV-head group) "
                      f"slices of the prefill workload ({done[0]} .. {done[-1]}), "
                      f"{flops / 1e9:.1f} GFLOP in {spent:.1f} s"}


def cpu_oracle_decode_baseline(d, budget_s=6.0):
    """The float64 decode oracle, as it stands, on whole requests of the
    decode workload (in request order) until ~budget_s; GB/s of the same
    algorithmic bytes the GPU figure counts."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    kc, vc = d.k_cache.cpu().numpy(), d.v_cache.cpu().numpy()
    ks, vs = d.k_scale.cpu().numpy(), d.v_scale.cpu().numpy()
    q, cu, bt, sl = d.q.cpu(), d.cu_seqlens_q.cpu(), d.block_table.cpu().numpy(), d.seq_lens.cpu()
    Hkv, D, Hq = kc.shape[1], kc.shape[3], q.shape[1]
    spent, done, nbytes = 0.0, [], 0
    for r in range(len(d.q_lens)):
        t0 = time.perf_counter()
        oracle.decode_paged(q, cu, kc, vc, bt, sl, d.scale, True, ks, vs, requests=[r])
        spent += time.perf_counter() - t0
        L = int(sl[r])
        nbytes += L * Hkv * (2 * D + 8) + d.q_lens[r] * Hq * D * 4 + math.ceil(L / d.block_size) * 4
        done.append(r)
        if spent >= budget_s:
            break
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 decode oracle on requests {done[0]}..{done[-1]} of the decode workload "
                      f"({nbytes / 1e6:.0f} MB of cache) in {spent:.1f} s"}


def decode_graph_us(fn, reps=50):
    """The decode layer (partials + reduce) captured once as a HIP graph and
    replayed; each of the first replays is checked against the eager result
    (with eager work between them) before the timed replays."""
    ref = fn().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("decode graph replay differs from the eager result")
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    return 1e3 * s.elapsed_time(e) / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true",
                    help="also time the 227K-context verify and the large-head prefill")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the hot path here is the "
              "one-GPU kernel; multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import causal_softmax_attention_amd as A
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = synth.varlen_8seq_window1024(device=dev)
    d = synth.decode_64req_fp8(device=dev)
    f_fwd, f_bwd, pairs = prefill_flops(x)
    dec_bytes = decode_bytes(d)
    print(f"[bench] prefill T={x.total_tokens} pairs={pairs} fwd={f_fwd:.3e} bwd={f_bwd:.3e} flop; "
          f"decode tokens={int(d.seq_lens.sum())} bytes={dec_bytes:.3e}", file=sys.stderr, flush=True)

    def fwd():
        return A.attn_fwd_varlen(x.q, x.k, x.v, x.cu_seqlens, x.max_seqlen, x.scale, x.window,
                                 x.sink, x.g)

    o, lse = fwd()

    def bwd():
        return A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale,
                                 x.window, x.sink, x.g)

    def bwd_fused():
        return A.attn_bwd_varlen(x.q, x.k, x.v, o, x.do, lse, x.cu_seqlens, x.max_seqlen, x.scale,
                                 x.window, x.sink, x.g, flags=A.ATTN_BWD_FUSED_DQ)

    dec_max_q, dec_max_len = d.max_seqlen_q, d.max_seq_len   # host values, read once

    def dec():
        return A.attn_decode_paged(d.q, d.cu_seqlens_q, dec_max_q, d.k_cache, d.v_cache,
                                   d.kv_dtype, d.k_scale, d.v_scale, d.block_table, d.seq_lens,
                                   dec_max_len, d.scale)

    tm = Timer()
    for _ in range(args.warmup):
        fwd(); bwd(); dec()
    torch.cuda.synchronize()
    tm = Timer()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tm.run("fwd", fwd)
        tm.run("bwd", bwd)
        tm.run("decode", dec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    # the decode layer as a HIP graph (the pages time decode that way), outside the step
    dec_graph_us = decode_graph_us(dec)
    # the fused-dQ variant of the backward, timed outside the step
    tf = Timer()
    bwd_fused()
    for _ in range(max(3, args.steps // 4)):
        tf.run("bwd_fused", bwd_fused)
    torch.cuda.synchronize()
    us = {k: tm.mean_us(k) for k in ("fwd", "bwd", "decode")}
    tf_fwd = f_fwd / (us["fwd"] * 1e-6) / 1e12
    tf_bwd = f_bwd / (us["bwd"] * 1e-6) / 1e12
    tf_fb = (f_fwd + f_bwd) / ((us["fwd"] + us["bwd"]) * 1e-6) / 1e12
    gbps = dec_bytes / (us["decode"] * 1e-6) / 1e9

    phases = {
        "fwd": dict(kernel="attn_fwd_varlen (gate prefix + forward tile loop)", bound="mfma",
                    achieved=tf_fwd, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s"),
        "bwd": dict(kernel="attn_bwd_varlen (gate prefix + pre + dK/dV pass + dQ pass + post)",
                    bound="mfma", achieved=tf_bwd, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s"),
        "decode": dict(kernel="attn_decode_paged (split-K partials + LSE reduce)", bound="hbm",
                       achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s"),
    }
    dom = max(us, key=us.get)
    roof = dict(phases[dom])
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["us_per_launch"] = us[dom]
    roof["traffic"] = stored_traffic({"fwd": "attn_fwd_varlen", "bwd": "attn_bwd_varlen",
                                      "decode": "attn_decode_paged"}[dom])
    for ph in phases.values():
        ph["frac"] = ph["achieved"] / ph["peak"]

    out = {
        "metric": "decode µs/layer + HBM GB/s; prefill fwd+bwd TFLOP/s vs MFMA peak",
        "value": tf_fb,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset)",
        "config": {
            "workload": "prefill fwd+bwd: 8 packed seqs (lengths U[256,4096], seed 2, T=%d), "
                        "32q/8kv heads, d 128, window 1024, sink, log gates; decode: 64 requests "
                        "(contexts U[1,32768], seed 3), 64q/4kv heads, d 128, page 16, "
                        "per-token fp8 e4m3fn KV, split-K + LSE reduce" % x.total_tokens,
            "global_batch": len(x.seqlens), "seq_len": x.max_seqlen, "parallelism": "single-gpu",
        },
        "prefill": {"fwd_us": us["fwd"], "bwd_us": us["bwd"],
                    "fwd_us_median": tm.median_us("fwd"), "bwd_us_median": tm.median_us("bwd"),
                    "bwd_path": "two-pass (deterministic)",
                    "bwd_fused_dq_us": tf.mean_us("bwd_fused"),
                    "bwd_fused_dq_tflops": f_bwd / (tf.mean_us("bwd_fused") * 1e-6) / 1e12,
                    "fwd_tflops": tf_fwd,
                    "bwd_tflops": tf_bwd, "fwdbwd_tflops": tf_fb,
                    "fwd_frac_of_mfma_peak": tf_fwd / MFMA_BF16_PEAK_TFLOPS,
                    "fwdbwd_frac_of_mfma_peak": tf_fb / MFMA_BF16_PEAK_TFLOPS,
                    "flops_fwd": f_fwd, "flops_bwd": f_bwd},
        "decode": {"us_per_layer": us["decode"], "us_per_layer_median": tm.median_us("decode"),
                   "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
                   "algorithmic_bytes": dec_bytes, "graph_us_per_layer": dec_graph_us,
                   "graph_GBps": dec_bytes / (dec_graph_us * 1e-6) / 1e9},
        "roofline": roof,
        "phases": phases,
    }

    if args.extra:
        extra = {}
        for kvd, tag in ((synth.KV_BF16, "bf16"), (synth.KV_FP8_E4M3FN, "fp8")):
            d4 = synth.verify_3x4_227k(kv_dtype=kvd, device=dev)
            mlen4 = d4.max_seq_len
            f = lambda: A.attn_decode_paged(d4.q, d4.cu_seqlens_q, 4, d4.k_cache, d4.v_cache, kvd,
                                            d4.k_scale, d4.v_scale, d4.block_table, d4.seq_lens,
                                            mlen4, d4.scale)
            for _ in range(3):
                f()
            t4 = Timer()
            for _ in range(20):
                t4.run("v", f)
            torch.cuda.synchronize()
            u = t4.mean_us("v")
            extra[f"verify_{tag}"] = {"us_per_layer": u, "GBps": decode_bytes(d4) / (u * 1e-6) / 1e9}
            del d4
        # decode with sink, 4096-token window and log gate on the 64-request decode cache
        df = synth.decode_64req_fp8(device=dev, with_sink=True, window=4096, with_gate=True)
        dmax = df.max_seq_len
        ff = lambda: A.attn_decode_paged(df.q, df.cu_seqlens_q, 1, df.k_cache, df.v_cache, df.kv_dtype,
                                         df.k_scale, df.v_scale, df.block_table, df.seq_lens, dmax, df.scale,
                                         sink=df.sink, window=df.window, g_cache=df.g_cache)
        for _ in range(3):
            ff()
        tf_ = Timer()
        for _ in range(20):
            tf_.run("f", ff)
        torch.cuda.synchronize()
        uf = tf_.mean_us("f")
        vis = [min(int(L), 4096) for L in df.seq_lens.tolist()]     # keys inside the window (1 query each)
        Hkv_, D_, Hq_ = df.k_cache.shape[1], df.k_cache.shape[3], df.q.shape[1]
        fbytes = sum(vis) * (Hkv_ * (2 * D_ + 8) + Hq_ * 4)          # fp8 K+V, two scales, gate per query head
        extra["decode_sink_window4096_gate"] = {"us_per_layer": uf, "GBps": fbytes / (uf * 1e-6) / 1e9,
                                                "algorithmic_bytes": fbytes}
        del df
        # per-token fp8 KV-cache write: a 32K-token prefill's keys and values
        xw = synth.kv_write_inputs(32768, 4, 128, 16, 2048 + 64, seed=1, skip_frac=0.0, device=dev)
        fw = lambda: A.attn_kv_cache_write_fp8(xw["k_new"], xw["v_new"], xw["slot_mapping"], xw["k_cache"],
                                               xw["v_cache"], xw["k_scale"], xw["v_scale"])
        for _ in range(3):
            fw()
        tw = Timer()
        for _ in range(20):
            tw.run("w", fw)
        torch.cuda.synchronize()
        uw = tw.mean_us("w")
        wbytes = 32768 * 4 * 2 * (2 * 128 + 128 + 4)    # bf16 in, fp8 codes + fp32 scale out
        extra["kv_cache_write_fp8"] = {"tokens": 32768, "kv_heads": 4, "head_dim": 128, "us": uw,
                                       "GBps": wbytes / (uw * 1e-6) / 1e9,
                                       "frac_of_hbm_peak": wbytes / (uw * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del xw
        # paged prefill: 4 chunks of 2048 new tokens over 4K-32K contexts, per-token fp8 cache
        dp = synth.prefill_paged_bench(device=dev)
        pmax, pq = dp.max_seq_len, dp.max_seqlen_q
        fp = lambda: A.attn_prefill_paged(dp.q, dp.cu_seqlens_q, pq, dp.k_cache, dp.v_cache, dp.kv_dtype,
                                          dp.k_scale, dp.v_scale, dp.block_table, dp.seq_lens, pmax, dp.scale)
        fp()
        tp = Timer()
        for _ in range(5):
            tp.run("p", fp)
        torch.cuda.synchronize()
        up = tp.mean_us("p")
        pfl = synth.paged_attention_flops(dp.seq_lens.tolist(), dp.q_lens, dp.q.shape[1], dp.q.shape[2])
        extra["prefill_paged_fp8"] = {"workload": "chunked prefill 4 x 2048 new tokens, contexts 4K-32K, "
                                                  "h64 kv4 d128 page 16, per-token fp8 KV",
                                      "us": up, "tflops": pfl / (up * 1e-6) / 1e12,
                                      "frac_of_bf16_mfma_peak": pfl / (up * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        del dp
        x5 = synth.varlen_4x8192_wide_heads(device=dev)
        f5f, f5b, _ = prefill_flops(x5)
        o5, l5 = A.attn_fwd_varlen(x5.q, x5.k, x5.v, x5.cu_seqlens, x5.max_seqlen, x5.scale, 0,
                                   x5.sink, x5.g)
        t5 = Timer()
        for _ in range(3):
            t5.run("f", lambda: A.attn_fwd_varlen(x5.q, x5.k, x5.v, x5.cu_seqlens, x5.max_seqlen,
                                                  x5.scale, 0, x5.sink, x5.g))
            t5.run("b", lambda: A.attn_bwd_varlen(x5.q, x5.k, x5.v, o5, x5.do, l5, x5.cu_seqlens,
                                                  x5.max_seqlen, x5.scale, 0, x5.sink, x5.g))
        torch.cuda.synchronize()
        extra["prefill_large_heads"] = {
            "fwd_us": t5.mean_us("f"), "bwd_us": t5.mean_us("b"),
            "fwd_tflops": f5f / (t5.mean_us("f") * 1e-6) / 1e12,
            "bwd_tflops": f5b / (t5.mean_us("b") * 1e-6) / 1e12}
        out["extra_workloads"] = extra

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_oracle_baseline(x)
        out["decode"]["cpu_oracle"] = cpu_oracle_decode_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
