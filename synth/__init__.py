"""Seeded synthetic inputs for the attention hot path.

This module only draws random inputs and lays them out; it holds none of the
attention arithmetic.  Both the CPU oracle (through the tests) and the HIP
path consume what it produces, so it must stay free of any step of the
method itself.

Shapes and value distributions follow the workloads described on the pages:
  * fla issue #1322, Description: dense and packed variable-length causal
    attention with GQA/MQA, unequal q/k and v head dims up to 512,
    logarithmic gates, sliding windows and a sink bias;
  * ROCm/aiter PR #6660, "Technical details" and "Test plan": paged decode
    over an fp8 e4m3 cache with one float32 K and one V scale per cached token
    laid out [num_blocks, num_kv_heads, block_size], token magnitudes that
    differ by up to 20x, NaN in unused scale slots, and short-query verify.

Small structural choices (sequence lengths, page permutation) are drawn with
``numpy.random.default_rng(seed)``; dense tensors with a seeded
``torch.Generator`` on the requested device, so the large decode caches can be
produced directly in device memory.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_E4M3FN_MAX = 448.0  # largest finite OCP e4m3fn value, used to size scales
FP8_POISON_BYTE = 0x7F  # an e4m3fn NaN code, written into unused cache slots
KV_BF16 = 0
KV_FP8_E4M3FN = 1


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, dtype=torch.float32):
    return torch.randn(shape, generator=gen, device=device, dtype=dtype)


# ----------------------------------------------------------------------------
# Prefill (packed variable-length) inputs
# ----------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    q: torch.Tensor            # bf16 [T, Hq, d_qk]
    k: torch.Tensor            # bf16 [T, Hkv, d_qk]
    v: torch.Tensor            # bf16 [T, Hkv, d_v]
    do: torch.Tensor           # bf16 [T, Hq, d_v]  (upstream gradient)
    cu_seqlens: torch.Tensor   # int32 [N+1]
    seqlens: list
    scale: float
    window: int                # <= 0: no window
    sink: Optional[torch.Tensor]  # fp32 [Hq] or None
    g: Optional[torch.Tensor]     # fp32 [T, Hq] log gates or None
    name: str = ""

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens)) if self.seqlens else 0

    def to(self, device) -> "PrefillInputs":
        mv = lambda t: None if t is None else t.to(device)
        return PrefillInputs(mv(self.q), mv(self.k), mv(self.v), mv(self.do),
                             mv(self.cu_seqlens), list(self.seqlens), self.scale,
                             self.window, mv(self.sink), mv(self.g), self.name)


def prefill_inputs(seqlens, Hq, Hkv, d_qk, d_v, *, seed, window=0,
                   with_sink=True, with_gate=True, scale=None,
                   device="cpu", name="") -> PrefillInputs:
    """q, k, v, dO ~ N(0,1) rounded to bf16 (round-to-nearest-even cast);
    sink ~ N(0,1); log gates g = log(sigmoid(N(3,1))) per token and query
    head (fla issue #1322 Description; gate and sink distribution as in the
    packed prefill workload of that feature set)."""
    seqlens = [int(x) for x in seqlens]
    T = int(sum(seqlens))
    gen = _gen(seed, device)
    q = _randn((T, Hq, d_qk), gen, device).to(torch.bfloat16)
    k = _randn((T, Hkv, d_qk), gen, device).to(torch.bfloat16)
    v = _randn((T, Hkv, d_v), gen, device).to(torch.bfloat16)
    do = _randn((T, Hq, d_v), gen, device).to(torch.bfloat16)
    sink = _randn((Hq,), gen, device) if with_sink else None
    g = None
    if with_gate:
        g = torch.nn.functional.logsigmoid(_randn((T, Hq), gen, device) + 3.0)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32),
                      device=device)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    return PrefillInputs(q, k, v, do, cu, seqlens, float(scale), int(window),
                         sink, g, name)


def dense_128_gqa4(device="cpu") -> PrefillInputs:
    """Dense causal fwd+bwd: one sequence of 128, 4 query heads over 1 KV head,
    head dim 64, sink per head, scale 1/8; no gate, no window."""
    return prefill_inputs([128], 4, 1, 64, 64, seed=1, window=0, with_sink=True,
                          with_gate=False, scale=1.0 / 8.0, device=device,
                          name="dense-128-gqa4-d64-sink")


def varlen_8seq_lengths():
    return [int(x) for x in np.random.default_rng(2).integers(256, 4097, 8)]


def varlen_8seq_window1024(device="cpu") -> PrefillInputs:
    """Packed varlen causal prefill: 8 sequences of length U[256, 4096]
    (seed 2), 32 query / 8 KV heads, head dim 128, window 1024, sink and
    log gates."""
    return prefill_inputs(varlen_8seq_lengths(), 32, 8, 128, 128, seed=2, window=1024,
                          with_sink=True, with_gate=True, device=device,
                          name="varlen-8seq-h32kv8-d128-w1024-sink-gate")


def varlen_4x8192_wide_heads(device="cpu") -> PrefillInputs:
    """Packed varlen fwd+bwd with large heads: 4 x 8192 tokens, 16 query /
    4 KV heads, d_qk 256, d_v 512, sinks and log gates, no window."""
    return prefill_inputs([8192] * 4, 16, 4, 256, 512, seed=5, window=0,
                          with_sink=True, with_gate=True, device=device,
                          name="varlen-4x8192-h16kv4-dqk256-dv512-sink-gate")


# ----------------------------------------------------------------------------
# Paged decode inputs
# ----------------------------------------------------------------------------
@dataclass
class DecodeInputs:
    q: torch.Tensor             # bf16 [Tq, Hq, D]
    cu_seqlens_q: torch.Tensor  # int32 [R+1]
    q_lens: list
    k_cache: torch.Tensor       # uint8 (fp8 codes) or bf16, [NB, Hkv, B, D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # fp32 [NB, Hkv, B] (fp8 only)
    v_scale: Optional[torch.Tensor]
    block_table: torch.Tensor   # int32 [R, max_pages]
    seq_lens: torch.Tensor      # int32 [R], KV length including new tokens
    kv_dtype: int               # KV_BF16 or KV_FP8_E4M3FN
    block_size: int
    scale: float
    name: str = ""
    unquantized_k: Optional[torch.Tensor] = field(default=None, repr=False)
    unquantized_v: Optional[torch.Tensor] = field(default=None, repr=False)
    sink: Optional[torch.Tensor] = None        # fp32 [Hq] sink logits, or None
    window: int = 0                            # sliding window (<= 0: none)
    g_cache: Optional[torch.Tensor] = None     # fp32 [NB, Hq, B] cumulative log gates, or None
    per_tensor: bool = False                   # fp8 with one K and one V scale ([1] each)

    @property
    def num_requests(self): return int(self.block_table.shape[0])
    @property
    def max_pages(self): return int(self.block_table.shape[1])
    @property
    def num_blocks(self): return int(self.k_cache.shape[0])
    @property
    def max_seqlen_q(self): return int(max(self.q_lens))
    @property
    def max_seq_len(self): return int(self.seq_lens.max().item())


def decode_inputs(seq_lens, q_lens, Hq, Hkv, D, B, *, kv_dtype, seed,
                  spread=20.0, spare_pages=64, device="cpu",
                  keep_unquantized=False, shuffle=True, name="",
                  window=0, with_sink=False, with_gate=False, per_tensor=False,
                  gate_slope=0.002) -> DecodeInputs:
    """A paged KV cache [NB, Hkv, B, D] with a shuffled page table.

    Values per (token, KV head) are N(0,1) * spread**u, u ~ U(0,1), drawn
    independently for K and V (the 20x token-magnitude spread of the aiter
    per-token-scale test plan).  For fp8 the cache is quantised per token and
    KV head with scale = amax/448 and a round-to-nearest-even cast to
    e4m3fn; unused scale slots hold NaN and unused data bytes a NaN code.  For
    bf16 unused slots hold bf16 NaN.  Spare pages that no request references
    are poisoned the same way.

    Optional decode features: ``with_sink`` draws sink logits N(0,1) per
    query head; ``window`` is passed through; ``with_gate`` fills a gate cache
    [NB, Hq, B] with a slowly falling sequence per (token, query head):
    G = -gate_slope * (token position) * r_h + 0.05 * N(0,1), r_h ~ U(0.5, 1.5)
    (any values are valid decode inputs; unused slots hold NaN);
    ``per_tensor`` (fp8) quantises each cache with one scale, the amax of its
    valid values / 448.
    """
    rng = np.random.default_rng(seed)
    seq_lens = [int(x) for x in seq_lens]
    q_lens = [int(x) for x in q_lens]
    assert len(seq_lens) == len(q_lens)
    assert all(1 <= n <= L for n, L in zip(q_lens, seq_lens))
    R = len(seq_lens)
    pages = [(L + B - 1) // B for L in seq_lens]
    used = int(sum(pages))
    NB = used + int(spare_pages)
    perm = rng.permutation(NB).astype(np.int32) if shuffle else np.arange(NB, dtype=np.int32)
    max_pages = max(pages)
    # Padding entries point at a spare (poisoned) page: never read by a
    # correct kernel, and NaN if one ever were.
    pad = int(perm[used]) if spare_pages > 0 else 0
    bt = np.full((R, max_pages), pad, dtype=np.int32)
    owner_len = np.zeros(NB, dtype=np.int64)   # valid slots in each page
    page_pos = np.zeros(NB, dtype=np.int64)    # index of the page within its request
    off = 0
    for r in range(R):
        ids = perm[off:off + pages[r]]
        bt[r, :pages[r]] = ids
        for p, pid in enumerate(ids):
            owner_len[pid] = min(B, seq_lens[r] - p * B)
            page_pos[pid] = p
        off += pages[r]

    gen = _gen(seed, device)
    Tq = int(sum(q_lens))
    q = _randn((Tq, Hq, D), gen, device).to(torch.bfloat16)

    valid = torch.from_numpy(np.arange(B)[None, :] < owner_len[:, None]).to(device)
    valid = valid[:, None, :].expand(NB, Hkv, B)          # [NB, Hkv, B]

    def draw():
        x = _randn((NB, Hkv, B, D), gen, device)
        if spread != 1.0:
            u = torch.rand((NB, Hkv, B, 1), generator=gen, device=device)
            x.mul_(torch.pow(torch.tensor(float(spread), device=device), u))
        return x

    def make(x):
        if kv_dtype == KV_FP8_E4M3FN and per_tensor:
            amax = torch.where(valid[..., None], x.abs(), torch.zeros_like(x)).amax()
            sc1 = (amax / FP8_E4M3FN_MAX).reshape(1).to(torch.float32)
            codes = (x / sc1).to(torch.float8_e4m3fn).view(torch.uint8)
            codes = torch.where(valid[..., None], codes,
                                torch.full_like(codes, FP8_POISON_BYTE))
            return codes.contiguous(), sc1.contiguous()
        if kv_dtype == KV_FP8_E4M3FN:
            amax = x.abs().amax(dim=-1)
            sc = torch.where(amax > 0, amax / FP8_E4M3FN_MAX, torch.ones_like(amax))
            codes = (x / sc[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
            codes = torch.where(valid[..., None], codes,
                                torch.full_like(codes, FP8_POISON_BYTE))
            sc = torch.where(valid, sc, torch.full_like(sc, float("nan")))
            return codes.contiguous(), sc.contiguous()
        data = x.to(torch.bfloat16)
        data = torch.where(valid[..., None], data,
                           torch.full_like(data, float("nan")))
        return data.contiguous(), None

    xk = draw()
    kc, ks = make(xk)
    if not keep_unquantized:
        del xk
        xk = None
    xv = draw()
    vc, vs = make(xv)
    if not keep_unquantized:
        del xv
        xv = None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32),
                      device=device)
    sink = _randn((Hq,), gen, device) if with_sink else None
    g_cache = None
    if with_gate:
        pos = torch.from_numpy(page_pos[:, None] * B + np.arange(B)[None, :]).to(device)   # [NB, B]
        rate = torch.rand((Hq,), generator=gen, device=device) + 0.5
        G = (-gate_slope * pos[:, None, :].to(torch.float32) * rate[None, :, None]
             + 0.05 * _randn((NB, Hq, B), gen, device))
        gvalid = torch.from_numpy(np.arange(B)[None, :] < owner_len[:, None]).to(device)[:, None, :]
        g_cache = torch.where(gvalid, G, torch.full_like(G, float("nan"))).contiguous()
    return DecodeInputs(q, cu, q_lens, kc, vc, ks, vs,
                        torch.from_numpy(bt).to(device),
                        torch.tensor(seq_lens, dtype=torch.int32, device=device),
                        int(kv_dtype), int(B), 1.0 / math.sqrt(D), name, xk, xv,
                        sink, int(window), g_cache, bool(per_tensor and kv_dtype == KV_FP8_E4M3FN))


def decode_64req_lengths():
    return [int(x) for x in np.random.default_rng(3).integers(1, 32769, 64)]


def decode_64req_fp8(device="cpu", **kw) -> DecodeInputs:
    """Paged single-query decode: 64 requests with contexts U[1, 32768]
    (seed 3), 64 query / 4 KV heads, D 128, page 16, per-token fp8."""
    L = decode_64req_lengths()
    return decode_inputs(L, [1] * len(L), 64, 4, 128, 16,
                         kv_dtype=KV_FP8_E4M3FN, seed=3, device=device,
                         name="decode-64req-ctx1-32768-h64kv4-d128-p16-fp8", **kw)


VERIFY_227K_SEQ_LENS = [226_944 + 1, 226_944 + 2, 226_944 + 4]


def verify_3x4_227k(kv_dtype=KV_FP8_E4M3FN, device="cpu", **kw) -> DecodeInputs:
    """Short-query verify: 3 requests x 4 query tokens over ~227K-token
    contexts ending 1, 2 and 4 tokens into the last 128-token page; 64 query /
    4 KV heads, D 128; bf16 or per-token fp8 KV (token magnitudes N(0,1))."""
    tag = "fp8" if kv_dtype == KV_FP8_E4M3FN else "bf16"
    return decode_inputs(VERIFY_227K_SEQ_LENS, [4, 4, 4], 64, 4, 128, 128,
                         kv_dtype=kv_dtype, seed=4, spread=1.0, device=device,
                         name=f"verify-3x4q-ctx227k-h64kv4-d128-p128-{tag}", **kw)


PREFILL_PAGED_NEW_TOKENS = 2048


def prefill_paged_bench(device="cpu", **kw) -> DecodeInputs:
    """Chunked prefill over the paged fp8 cache: 4 requests, each adding 2048
    new tokens to a context whose total length is drawn uniformly in
    [4096, 32768] (seeded); 64 query / 4 KV heads, D 128, page 16, per-token
    fp8 K/V with the 20x token-magnitude spread, shuffled page table."""
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(4096, 32769, 4)]
    return decode_inputs(lens, [PREFILL_PAGED_NEW_TOKENS] * 4, 64, 4, 128, 16,
                         kv_dtype=KV_FP8_E4M3FN, seed=12, device=device,
                         name="chunked-prefill-4x2048new-ctx4k-32k-h64kv4-d128-p16-fp8", **kw)


def paged_attention_flops(seq_lens, q_lens, Hq, D, window=0):
    """Algorithmic flops of causal paged attention: 4 D per visible
    (query row, key) pair (QK^T and PV, one multiply-add each)."""
    total = 0
    for L, n in zip(seq_lens, q_lens):
        pos = np.arange(int(L) - int(n), int(L), dtype=np.int64)
        vis = pos + 1 if window <= 0 else np.minimum(pos + 1, window)
        total += int(vis.sum())
    return 4.0 * D * Hq * total


# ----------------------------------------------------------------------------
# Split-K partial tensors (for the reduce entry point on its own)
# ----------------------------------------------------------------------------
def partials_inputs(rows, S, Dv, *, seed, empty_frac=0.25, device="cpu"):
    """Random (acc, m, l) partials; a fraction of (row, split) entries are
    empty (m = -inf, and acc / l hold NaN so any read of them shows).  Every
    row keeps at least one non-empty split unless ``empty_frac`` is 1."""
    gen = _gen(seed, device)
    m = _randn((rows, S), gen, device) * 4.0
    l = torch.rand((rows, S), generator=gen, device=device) * 50.0 + 1.0
    acc = _randn((rows, S, Dv), gen, device) * l[..., None]
    empty = torch.rand((rows, S), generator=gen, device=device) < empty_frac
    if empty_frac < 1.0:
        keep = torch.randint(0, S, (rows,), generator=gen, device=device)
        empty[torch.arange(rows, device=device), keep] = False
    m = torch.where(empty, torch.full_like(m, float("-inf")), m)
    l = torch.where(empty, torch.full_like(l, float("nan")), l)
    acc = torch.where(empty[..., None], torch.full_like(acc, float("nan")), acc)
    return acc.contiguous(), m.contiguous(), l.contiguous()


# ----------------------------------------------------------------------------
# KV-cache write inputs
# ----------------------------------------------------------------------------
def kv_write_inputs(N, Hkv, D, B, NB, *, seed, skip_frac=0.1, zero_rows=1, device="cpu"):
    """New tokens for a paged fp8 cache write.

    k_new, v_new bf16 [N, Hkv, D] with per-(token, head) magnitudes varying up
    to 20x (N(0,1) * 20^u, as in the decode caches); ``zero_rows`` (token,
    head) rows are all zeros.  slot_mapping int32 [N]: distinct slots drawn
    from the NB * B slots, a fraction ``skip_frac`` replaced by -1 (padding).
    The caches start poisoned (0x7F bytes, NaN scales) so that any slot the
    write should not touch shows."""
    gen = _gen(seed, "cpu")
    mag = torch.pow(torch.tensor(20.0), torch.rand((N, Hkv, 1), generator=gen))
    k = (_randn((N, Hkv, D), gen, "cpu") * mag).to(torch.bfloat16)
    mag = torch.pow(torch.tensor(20.0), torch.rand((N, Hkv, 1), generator=gen))
    v = (_randn((N, Hkv, D), gen, "cpu") * mag).to(torch.bfloat16)
    for i in range(min(zero_rows, N * Hkv)):
        t, h = divmod((i * 7919) % (N * Hkv), Hkv)
        k[t, h] = 0
        v[(t + 1) % N, h] = 0
    assert N <= NB * B
    slots = torch.randperm(NB * B, generator=gen)[:N].to(torch.int32)
    skip = torch.rand((N,), generator=gen) < skip_frac
    slots = torch.where(skip, torch.full_like(slots, -1), slots)
    k_cache = torch.full((NB, Hkv, B, D), 0x7F, dtype=torch.uint8)
    v_cache = k_cache.clone()
    k_scale = torch.full((NB, Hkv, B), float("nan"), dtype=torch.float32)
    v_scale = k_scale.clone()
    out = dict(k_new=k, v_new=v, slot_mapping=slots, k_cache=k_cache, v_cache=v_cache,
               k_scale=k_scale, v_scale=v_scale)
    return {n: t.to(device).contiguous() for n, t in out.items()}
