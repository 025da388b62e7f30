"""The allocation-free decode entry point (attn_decode_paged_noalloc) against
the workspace one (attn_decode_paged), both called through the C ABI.

Two calls in a row share the library's per-GPU scratch, the second with a
smaller input; each must match the workspace entry point's output and lse
(same kernels, same grid: bit for bit, and within the 5e-3 relative-RMS
bar).  (The rejection of calls whose partials do not fit the scratch is
pure host arithmetic, tested without a GPU in test_boundary.py.)
"""
import ctypes
import sys

import pytest
import torch

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


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _common_args(d):
    NB, Hkv, B, D = d.k_cache.shape
    Hq = d.q.shape[1]
    R = d.seq_lens.numel()
    return [_p(d.q), _p(d.cu_seqlens_q), R, int(d.max_seqlen_q), _p(d.k_cache), _p(d.v_cache),
            int(d.kv_dtype), _p(d.k_scale), _p(d.v_scale), _p(d.block_table), d.block_table.shape[1],
            _p(d.seq_lens), int(d.max_seq_len), NB, B, Hq, Hkv, D, ctypes.c_float(d.scale), 0]


def _with_workspace(A, d):
    L = A.library
    R, (NB, Hkv, B, D), Hq = d.seq_lens.numel(), d.k_cache.shape, d.q.shape[1]
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device=DEV)
    n = L.attn_decode_workspace_size(R, int(d.max_seqlen_q), int(d.max_seq_len), Hq, Hkv, D, B, 0)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    st = L.attn_decode_paged(*_common_args(d), _p(out), _p(lse), _p(ws), n, None)
    assert st == 0, L.attn_last_error()
    return out, lse


def _no_alloc(A, d):
    L = A.library
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    st = L.attn_decode_paged_noalloc(*_common_args(d), _p(out), _p(lse), None)
    assert st == 0, L.attn_last_error()
    return out, lse


def _f(t):
    return t.detach().float().cpu().double().numpy()


def test_noalloc_decode_matches_workspace_decode_twice(A):
    # call 1: per-token fp8 cache, 24 single-token requests (balanced split)
    big = synth.decode_inputs([int(x) for x in torch.randint(1, 6000, (24,), generator=torch.Generator().manual_seed(5))],
                              [1] * 24, 64, 4, 128, 16, kv_dtype=synth.KV_FP8_E4M3FN, seed=21, device=DEV,
                              spare_pages=8)
    # call 2, smaller: 4-token verify of 3 requests over a bf16 cache
    small = synth.decode_inputs([900, 37, 2100], [4, 4, 4], 64, 4, 128, 32, kv_dtype=synth.KV_BF16, seed=22,
                                device=DEV, spare_pages=2)
    for name, d in (("fp8 24x1", big), ("bf16 3x4", small)):
        _say(f"[case] no-alloc decode {name}")
        ro, rl = _with_workspace(A, d)
        no, nl = _no_alloc(A, d)
        torch.cuda.synchronize()
        err = rel_rms(_f(no), _f(ro))
        _say(f"    out rel_rms vs workspace entry point = {err:.3e}")
        assert err <= 5e-3
        assert torch.equal(no, ro)
        assert torch.equal(nl, rl)
