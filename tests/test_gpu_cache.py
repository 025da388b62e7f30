"""GPU parity of the per-token fp8 KV-cache write against the oracle.

Codes and scales are integer / exactly-decided results: the bar is bit
equality (both sides take every floating-point decision in float32).  Slots
the write must not touch keep their poison.  End to end, decode over a cache
written by the kernel matches the float64 decode oracle on that cache."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.util import rel_rms

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def A():
    import causal_softmax_attention_amd as A
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return A


CASES = [
    # N, Hkv, D, B, NB
    (1, 1, 128, 16, 1),
    (37, 4, 128, 16, 8),
    (200, 8, 64, 32, 10),
    (513, 4, 128, 128, 6),
    (4096, 4, 128, 16, 300),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}-h{c[1]}-d{c[2]}-p{c[3]}")
def test_cache_write_bit_exact(A, case):
    N, Hkv, D, B, NB = case
    _say(f"[case] kv cache write N={N} Hkv={Hkv} D={D} B={B} NB={NB}")
    x = synth.kv_write_inputs(N, Hkv, D, B, NB, seed=N + D, device=DEV)
    ref = oracle.cache_write_fp8(x["k_new"].float().cpu().numpy(), x["v_new"].float().cpu().numpy(),
                                 x["slot_mapping"].cpu().numpy(), x["k_cache"].cpu().numpy(),
                                 x["v_cache"].cpu().numpy(), x["k_scale"].cpu().numpy(),
                                 x["v_scale"].cpu().numpy())
    A.attn_kv_cache_write_fp8(x["k_new"], x["v_new"], x["slot_mapping"], x["k_cache"], x["v_cache"],
                              x["k_scale"], x["v_scale"])
    torch.cuda.synchronize()
    got = [x["k_cache"].cpu().numpy(), x["v_cache"].cpu().numpy(), x["k_scale"].cpu().numpy(),
           x["v_scale"].cpu().numpy()]
    for name, g, r in zip(("k codes", "v codes"), got[:2], ref[:2]):
        bad = int(np.count_nonzero(g != r))
        _say(f"    {name}: {bad} mismatching bytes")
        assert bad == 0
    for name, g, r in zip(("k scales", "v scales"), got[2:], ref[2:]):
        same = (g == r) | (np.isnan(g) & np.isnan(r))     # untouched slots keep NaN
        assert same.all(), name


def test_cache_write_then_decode(A):
    """A cache filled by the kernel decodes like the oracle's decode of it."""
    R, Hq, Hkv, D, B = 3, 16, 2, 128, 16
    seq_lens = [37, 300, 1029]
    NB = sum((L + B - 1) // B for L in seq_lens) + 4
    gen = torch.Generator().manual_seed(7)
    # pages in a shuffled order; tokens of request r fill their pages in order
    perm = torch.randperm(NB, generator=gen).tolist()
    bt = torch.zeros((R, max((L + B - 1) // B for L in seq_lens)), dtype=torch.int32)
    slots, off = [], 0
    for r, L in enumerate(seq_lens):
        npg = (L + B - 1) // B
        pages = perm[off:off + npg]; off += npg
        bt[r, :npg] = torch.tensor(pages, dtype=torch.int32)
        slots += [pages[j // B] * B + j % B for j in range(L)]
    N = len(slots)
    x = synth.kv_write_inputs(N, Hkv, D, B, NB, seed=5, skip_frac=0.0, device=DEV)
    x["slot_mapping"] = torch.tensor(slots, dtype=torch.int32, device=DEV)
    A.attn_kv_cache_write_fp8(x["k_new"], x["v_new"], x["slot_mapping"], x["k_cache"], x["v_cache"],
                              x["k_scale"], x["v_scale"])
    q = (torch.randn((R, Hq, D), generator=gen)).to(torch.bfloat16).to(DEV)
    cu = torch.arange(R + 1, dtype=torch.int32, device=DEV)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    out = A.attn_decode_paged(q, cu, 1, x["k_cache"], x["v_cache"], A.ATTN_DTYPE_FP8_E4M3FN,
                              x["k_scale"], x["v_scale"], bt.to(DEV), sl, max(seq_lens), 0.088)
    torch.cuda.synchronize()
    ro, _ = oracle.decode_paged(q, cu, x["k_cache"], x["v_cache"], bt.to(DEV), sl, 0.088, True,
                                x["k_scale"], x["v_scale"])
    err = rel_rms(out.float().cpu().double().numpy(), ro)
    _say(f"[case] write+decode rel_rms={err:.2e}")
    assert err <= 5e-3
