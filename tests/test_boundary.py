"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects every malformed or unsupported argument with
its status code before anything is launched (so these calls never reach the
GPU).  Pointers here are fake but aligned, non-null addresses: each call is
built to fail validation, which never dereferences them."""
import ctypes
import os
import re

import pytest

import causal_softmax_attention_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = A.library
P = ctypes.c_void_p(0x10000)          # aligned stand-in pointer (never read)
P_ODD = ctypes.c_void_p(0x10004)      # 4-byte but not 16-byte aligned
NULL = None
OK, INVALID, UNSUPPORTED = 0, -1, -2


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_all_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(A.lib_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"


def test_status_strings_and_version():
    assert L.attn_status_string(0) == b"ok"
    assert L.attn_status_string(-2) == b"unsupported configuration"
    assert L.attn_status_string(123) == b"unknown status"
    assert b"gfx950" in L.attn_version()


def _decode(**kw):
    a = dict(q=P, cu=P, R=2, maxq=1, kc=P, vc=P, kvd=A.ATTN_DTYPE_FP8_E4M3FN, ks=P, vs=P, bt=P,
             maxp=8, sl=P, maxsl=128, nb=16, B=16, Hq=64, Hkv=4, D=128, scale=0.1, split=0,
             out=P, lse=NULL, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.attn_decode_paged(a["q"], a["cu"], a["R"], a["maxq"], a["kc"], a["vc"], a["kvd"], a["ks"],
                               a["vs"], a["bt"], a["maxp"], a["sl"], a["maxsl"], a["nb"], a["B"], a["Hq"],
                               a["Hkv"], a["D"], a["scale"], a["split"], a["out"], a["lse"], a["ws"],
                               a["wsb"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(maxq=5), UNSUPPORTED, "prefill"),
    (dict(maxq=0), INVALID, "max_seqlen_q"),
    (dict(ks=NULL), UNSUPPORTED, "per-token"),
    (dict(vs=NULL), UNSUPPORTED, "per-token"),
    (dict(kvd=A.ATTN_DTYPE_BF16), UNSUPPORTED, "only read with an fp8"),
    (dict(kvd=7), UNSUPPORTED, "kv_dtype"),
    (dict(D=96), UNSUPPORTED, "head_dim"),
    (dict(D=256), UNSUPPORTED, "head_dim"),
    (dict(B=24), UNSUPPORTED, "block_size"),
    (dict(Hq=60, Hkv=8), INVALID, "multiple"),
    (dict(Hq=128, Hkv=2, maxq=4), UNSUPPORTED, "exceeds 64"),
    (dict(split=48), INVALID, "multiple of"),
    (dict(split=16384), UNSUPPORTED, "exceeds"),
    (dict(maxp=4), INVALID, "cannot hold"),
    (dict(q=NULL), INVALID, "q is NULL"),
    (dict(kc=P_ODD), INVALID, "aligned"),
    (dict(wsb=16, maxsl=4096, maxp=256), INVALID, "workspace too small"),
    (dict(maxsl=(1 << 30) + 1, maxp=(1 << 26) + 1), UNSUPPORTED, "exceeds 2^30"),
    (dict(R=-1), INVALID, "negative"),
    (dict(scale=float("nan")), INVALID, "finite"),
])
def test_decode_validation(kw, code, msg):
    st = _decode(**kw)
    assert st == code
    assert msg in L.attn_last_error().decode()


def test_decode_empty_batch_is_a_no_op():
    assert _decode(R=0) == OK


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kvd", [A.ATTN_DTYPE_BF16, A.ATTN_DTYPE_FP8_E4M3FN])
def test_decode_accepts_head_dims_64_and_128_for_both_caches(D, kvd):
    # past the head-dim and cache-dtype checks, stopped by a NULL output
    sc = P if kvd == A.ATTN_DTYPE_FP8_E4M3FN else NULL
    assert _decode(D=D, kvd=kvd, ks=sc, vs=sc, out=NULL) == INVALID
    assert "out is NULL" in L.attn_last_error().decode()


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, cu=P, N=2, maxs=64, T=100, Hq=8, Hkv=2, dqk=128, dv=128, scale=0.1, W=0,
             sink=NULL, g=NULL, o=P, lse=P, ws=NULL, wsb=0)
    a.update(kw)
    return L.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cu"], a["N"], a["maxs"], a["T"], a["Hq"], a["Hkv"],
                             a["dqk"], a["dv"], a["scale"], a["W"], a["sink"], a["g"], a["o"], a["lse"],
                             a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dqk=96, dv=96), UNSUPPORTED, "head dims"),
    (dict(dqk=512, dv=512), UNSUPPORTED, "head dims"),
    (dict(dqk=32, dv=64), UNSUPPORTED, "head dims"),
    (dict(dqk=128, dv=1024), UNSUPPORTED, "head dims"),
    (dict(dqk=256, dv=96), UNSUPPORTED, "head dims"),
    (dict(Hq=6, Hkv=4), INVALID, "multiple"),
    (dict(Hkv=0), INVALID, "positive"),
    (dict(maxs=0), INVALID, "max_seqlen"),
    (dict(maxs=101), INVALID, "max_seqlen"),
    (dict(q=NULL), INVALID, "q is NULL"),
    (dict(v=P_ODD), INVALID, "aligned"),
    (dict(o=NULL), INVALID, "o is NULL"),
    (dict(g=P, wsb=0), INVALID, "workspace too small"),
    (dict(scale=float("inf")), INVALID, "finite"),
    (dict(scale=0.0), INVALID, "positive"),
    (dict(scale=-0.1), INVALID, "positive"),
    (dict(N=70000), UNSUPPORTED, "num_seqs"),
])
def test_forward_validation(kw, code, msg):
    assert _fwd(**kw) == code
    assert msg in L.attn_last_error().decode()


# Every (d_qk, d_v) pair with d_qk in {64, 128, 256} and d_v in {64, 128,
# 256, 512} passes the head-dim check: each call is then stopped by a check
# that runs after it (a NULL output), never by the head dims.
HEAD_DIM_PAIRS = [(a, b) for a in (64, 128, 256) for b in (64, 128, 256, 512)]


@pytest.mark.parametrize("dqk,dv", HEAD_DIM_PAIRS)
def test_forward_accepts_every_head_dim_pair(dqk, dv):
    assert _fwd(dqk=dqk, dv=dv, o=NULL) == INVALID
    assert "o is NULL" in L.attn_last_error().decode()


def test_forward_empty_is_a_no_op():
    assert _fwd(N=0, T=0, maxs=0) == OK
    assert _fwd(T=0) == OK


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, cu=P, N=2, maxs=64, T=100, Hq=8, Hkv=2, dqk=128, dv=128,
             scale=0.1, W=0, sink=NULL, g=NULL, dq=P, dk=P, dv_=P, ds=NULL, dg=NULL, flags=0, ws=P, wsb=0)
    a.update(kw)
    return L.attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["cu"], a["N"], a["maxs"],
                             a["T"], a["Hq"], a["Hkv"], a["dqk"], a["dv"], a["scale"], a["W"], a["sink"],
                             a["g"], a["dq"], a["dk"], a["dv_"], a["ds"], a["dg"], a["flags"], a["ws"],
                             a["wsb"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(sink=P), INVALID, "dsink must be given"),
    (dict(ds=P), INVALID, "dsink must be given"),
    (dict(g=P), INVALID, "dg must be given"),
    (dict(flags=3), INVALID, "exclude each other"),
    (dict(flags=8), INVALID, "unknown flags"),
    (dict(flags=6), INVALID, "ATTN_BWD_RECOMPUTE_DQ belongs"),
    (dict(flags=2, dqk=256, dv=512), UNSUPPORTED, "fused-dQ"),
    (dict(do=NULL), INVALID, "dO is NULL"),
    (dict(wsb=64), INVALID, "workspace too small"),
    (dict(dqk=64, dv=96), UNSUPPORTED, "head dims"),
    (dict(dqk=512, dv=128), UNSUPPORTED, "head dims"),
    (dict(flags=2, dqk=256, dv=64), UNSUPPORTED, "fused-dQ"),
])
def test_backward_validation(kw, code, msg):
    assert _bwd(**kw) == code
    assert msg in L.attn_last_error().decode()


@pytest.mark.parametrize("dqk,dv", HEAD_DIM_PAIRS)
@pytest.mark.parametrize("flags", [0, 1, 2, 4, 5])
def test_backward_accepts_every_head_dim_pair(dqk, dv, flags):
    # the fused-dQ path (flag 2) covers d_qk <= 128; the two-pass path all pairs
    rc = _bwd(dqk=dqk, dv=dv, flags=flags, do=NULL)
    if flags == 2 and dqk > 128:
        assert rc == UNSUPPORTED and "fused-dQ" in L.attn_last_error().decode()
    else:
        assert rc == INVALID and "dO is NULL" in L.attn_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dv=96), UNSUPPORTED, "head_dim_v"),
    (dict(S=0), INVALID, "num_splits"),
    (dict(dt=7), UNSUPPORTED, "out_dtype"),
    (dict(acc=NULL), INVALID, "acc is NULL"),
    (dict(rows=-3), INVALID, "negative"),
])
def test_reduce_validation(kw, code, msg):
    a = dict(acc=P, m=P, l=P, rows=10, S=4, dv=128, out=P, dt=A.ATTN_DTYPE_FP32, lse=NULL)
    a.update(kw)
    st = L.attn_splitk_reduce(a["acc"], a["m"], a["l"], a["rows"], a["S"], a["dv"], a["out"], a["dt"],
                              a["lse"], NULL)
    assert st == code
    assert msg in L.attn_last_error().decode()


def test_workspace_sizes():
    # forward: gate prefix only
    assert A.attn_fwd_workspace_size(1000, 8, False) == 0
    assert A.attn_fwd_workspace_size(1000, 8, True) >= 1000 * 8 * 4
    # backward: the fused path holds an fp32 dQ accumulator; the two-pass one,
    # for d_v 512 and for d_qk 256 with d_v 128 / 256, stores dS (bf16 tiles
    # of 32 rows x 16 keys for every (row tile, key block) in the band, plus
    # fp32 row sums with a gate) unless told to recompute; other head dims
    # recompute
    rec = A.attn_bwd_workspace_size(1000, 2, 600, 8, 128, 128, 0, True, True, 0)
    fused = A.attn_bwd_workspace_size(1000, 2, 600, 8, 128, 128, 0, True, True, A.ATTN_BWD_FUSED_DQ)
    assert fused >= 1000 * 8 * 128 * 4 > rec
    for dqk, dv in ((128, 256), (256, 64), (64, 64)):
        assert A.attn_bwd_workspace_size(1000, 2, 600, 8, dqk, dv, 0, True, True, 0) == rec
    for dqk, dv in ((64, 512), (128, 512), (256, 128), (256, 256)):
        assert A.attn_bwd_workspace_size(1000, 2, 600, 8, dqk, dv, 0, True, True, 0) > rec
    assert A.attn_bwd_workspace_size(1000, 2, 600, 8, 256, 512, 0, True, True, A.ATTN_BWD_RECOMPUTE_DQ) == rec
    stored = A.attn_bwd_workspace_size(1000, 2, 600, 8, 256, 512, 0, True, True, 0)
    # 1000 // 32 + 2 + 1 row tiles, 2 * ceil(600 / 32) slots, 1 KB + 128 B each
    assert stored >= rec + 8 * (1000 // 32 + 3) * 38 * (1024 + 128)
    assert A.attn_bwd_workspace_size(1000, 2, 600, 8, 256, 256, 0, True, True,
                                     A.ATTN_BWD_DETERMINISTIC) == stored
    # a window bounds the slots per row tile: 2 + (W + 14) // 16
    win = A.attn_bwd_workspace_size(1000, 2, 600, 8, 256, 512, 64, True, True, 0)
    assert rec + 8 * 34 * 6 * 1024 <= win < stored
    # without a gate, no row sums
    assert A.attn_bwd_workspace_size(1000, 2, 600, 8, 256, 512, 0, False, True, 0) < stored
    # past 32 GiB of store the dQ pass recomputes: the size falls back to the
    # recomputing layout, also where the exact byte count would pass 2^64
    big = A.attn_bwd_workspace_size(2**31 - 1, 1, 2**31 - 1, 64, 256, 512, 0, True, True, 0)
    big_rec = A.attn_bwd_workspace_size(2**31 - 1, 1, 2**31 - 1, 64, 256, 512, 0, True, True,
                                        A.ATTN_BWD_RECOMPUTE_DQ)
    assert big == big_rec > 0
    mid = A.attn_bwd_workspace_size(131072, 1, 131072, 16, 256, 512, 0, True, True, 0)
    assert mid == A.attn_bwd_workspace_size(131072, 1, 131072, 16, 256, 512, 0, True, True,
                                            A.ATTN_BWD_RECOMPUTE_DQ)
    # sizes whose partials would pass 2^60 bytes (where exact products could
    # wrap) are reported as SIZE_MAX, which no workspace matches
    M = 2**31 - 1
    assert A.attn_decode_workspace_size(M, 4, M, 64, 4, 128, 16, 0) == 2**64 - 1
    assert A.attn_prefill_paged_workspace_size(M, M, M, 64, 4, 128, 16, 0) == 2**64 - 1
    # decode: partials for every (query row, split)
    ws = A.attn_decode_workspace_size(64, 1, 32768, 64, 4, 128, 16, 1024)
    assert ws >= 64 * 64 * 32 * 128 * 4
    assert A.attn_decode_workspace_size(64, 1, 32768, 64, 4, 128, 16, 0) > 0


def test_python_wrapper_rejects_strided_and_wrong_dtype():
    import torch
    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(10, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="contiguous"):
        A.attn_fwd_varlen(q.transpose(0, 1), k, k, cu, 10)
    with pytest.raises(ValueError, match="bfloat16"):
        A.attn_fwd_varlen(q.float(), k, k, cu, 10)
    with pytest.raises(ValueError, match="int32"):
        A.attn_fwd_varlen(q, k, k, cu.long(), 10)


def _kvw(**kw):
    a = dict(k=P, v=P, slots=P, N=4, H=4, D=128, kc=P, vc=P, ks=P, vs=P, NB=8, B=16)
    a.update(kw)
    return L.attn_kv_cache_write_fp8(a["k"], a["v"], a["slots"], a["N"], a["H"], a["D"], a["kc"], a["vc"],
                                     a["ks"], a["vs"], a["NB"], a["B"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(N=-1), INVALID, "negative"),
    (dict(H=0), INVALID, "num_kv_heads"),
    (dict(D=96), UNSUPPORTED, "head_dim"),
    (dict(B=24), UNSUPPORTED, "block_size"),
    (dict(k=NULL), INVALID, "k_new is NULL"),
    (dict(slots=NULL), INVALID, "slot_mapping is NULL"),
    (dict(ks=NULL), INVALID, "k_scale is NULL"),
    (dict(k=P_ODD), INVALID, "aligned"),
    (dict(NB=1 << 28, B=128), UNSUPPORTED, "int32 slot range"),
])
def test_kv_cache_write_validation(kw, code, msg):
    st = _kvw(**kw)
    assert st == code
    assert msg in L.attn_last_error().decode()


def test_kv_cache_write_empty_is_a_no_op():
    assert _kvw(N=0, k=NULL, v=NULL, slots=NULL) == OK


def _decode_ext(**kw):
    a = dict(q=P, cu=P, R=2, maxq=1, kc=P, vc=P, kvd=A.ATTN_DTYPE_FP8_E4M3FN, ks=P, vs=P, pt=0, bt=P,
             maxp=8, sl=P, maxsl=128, nb=16, B=16, Hq=64, Hkv=4, D=128, scale=0.1, sink=NULL, W=0,
             gc=NULL, split=0, out=P, lse=NULL, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.attn_decode_paged_ext(a["q"], a["cu"], a["R"], a["maxq"], a["kc"], a["vc"], a["kvd"], a["ks"],
                                   a["vs"], a["pt"], a["bt"], a["maxp"], a["sl"], a["maxsl"], a["nb"], a["B"],
                                   a["Hq"], a["Hkv"], a["D"], a["scale"], a["sink"], a["W"], a["gc"],
                                   a["split"], a["out"], a["lse"], a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(pt=2), INVALID, "per_tensor_scales"),
    (dict(pt=1, kvd=A.ATTN_DTYPE_BF16, ks=NULL, vs=NULL), UNSUPPORTED, "per-tensor scales need an fp8"),
    (dict(sink=ctypes.c_void_p(0x10002)), INVALID, "sink is not 4-byte aligned"),
    (dict(gc=P_ODD), INVALID, "g_cache is not 16-byte aligned"),
    (dict(gc=P, pt=1, nb=1 << 22, B=128, Hq=64), UNSUPPORTED, "gate cache larger than 4 GiB"),
    (dict(nb=1 << 23, B=128, Hkv=8, Hq=64), UNSUPPORTED, "per-token scale arrays larger than 4 GiB"),
])
def test_decode_ext_validation(kw, code, msg):
    st = _decode_ext(**kw)
    assert st == code
    assert msg in L.attn_last_error().decode()


def _prefill(**kw):
    a = dict(q=P, cu=P, R=2, maxq=512, kc=P, vc=P, kvd=A.ATTN_DTYPE_FP8_E4M3FN, ks=P, vs=P, pt=0, bt=P,
             maxp=64, sl=P, maxsl=1024, nb=128, B=16, Hq=64, Hkv=4, D=128, scale=0.1, sink=NULL, win=0,
             g=NULL, split=0, out=P, lse=NULL, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.attn_prefill_paged(a["q"], a["cu"], a["R"], a["maxq"], a["kc"], a["vc"], a["kvd"], a["ks"],
                                a["vs"], a["pt"], a["bt"], a["maxp"], a["sl"], a["maxsl"], a["nb"], a["B"],
                                a["Hq"], a["Hkv"], a["D"], a["scale"], a["sink"], a["win"], a["g"],
                                a["split"], a["out"], a["lse"], a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(maxq=0), INVALID, "max_seqlen_q"),
    (dict(ks=NULL), UNSUPPORTED, "per-token"),
    (dict(kvd=A.ATTN_DTYPE_BF16), UNSUPPORTED, "only read with an fp8"),
    (dict(D=256), UNSUPPORTED, "head_dim"),
    (dict(B=24), UNSUPPORTED, "block_size"),
    (dict(Hq=60, Hkv=8), INVALID, "multiple"),
    (dict(split=48), INVALID, "multiple of"),
    (dict(maxp=4), INVALID, "cannot hold"),
    (dict(q=NULL), INVALID, "q is NULL"),
    (dict(split=32, wsb=16), INVALID, "workspace too small"),
    (dict(R=1 << 10, maxq=1 << 10, split=32, maxsl=1 << 20, maxp=1 << 16, wsb=1 << 62), UNSUPPORTED,
     "work items"),
    (dict(pt=2), INVALID, "per_tensor_scales"),
    (dict(g=P, Hq=128, Hkv=1), UNSUPPORTED, "at most 64 query heads"),
])
def test_prefill_validation(kw, code, msg):
    st = _prefill(**kw)
    assert st == code
    assert msg in L.attn_last_error().decode()


def test_prefill_workspace_sizes():
    # enough query blocks for one segment per block: no partials, no workspace
    assert A.attn_prefill_paged_workspace_size(2, 4096, 8192, 64, 4, 128, 16) == 0
    # a short chunk over a long context: split-K partials
    n = A.attn_prefill_paged_workspace_size(1, 8, 200000, 64, 4, 128, 128)
    assert n >= 1 * 8 * 64 * 2 * (128 + 2) * 4
    # an explicit split of the whole context is one segment as well
    assert A.attn_prefill_paged_workspace_size(1, 8, 1000, 64, 4, 128, 16, 1024) == 0


# ---------------------------------------------------------------------------
# allocation-free decode: a call whose partials exceed the scratch is
# rejected by arithmetic alone, before any runtime call (this machine has no
# GPU, so reaching the runtime would give ATTN_ERR_HIP instead)
def _decode_noalloc(**kw):
    a = dict(q=P, cu=P, R=64, maxq=4, kc=P, vc=P, kvd=A.ATTN_DTYPE_FP8_E4M3FN, ks=P, vs=P, bt=P, maxp=2048,
             sl=P, maxsl=32768, nb=200000, B=16, Hq=64, Hkv=4, D=128, scale=0.1, split=512, out=P, lse=NULL)
    a.update(kw)
    return L.attn_decode_paged_noalloc(a["q"], a["cu"], a["R"], a["maxq"], a["kc"], a["vc"], a["kvd"],
                                       a["ks"], a["vs"], a["bt"], a["maxp"], a["sl"], a["maxsl"], a["nb"],
                                       a["B"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["split"], a["out"],
                                       a["lse"], NULL)


def test_noalloc_decode_rejects_calls_beyond_the_scratch():
    # 64 requests x 4 tokens x 64 heads x 64 segments of 512 keys: 16384 rows
    # x 64 partials x 520 bytes, far beyond the scratch
    assert _decode_noalloc() == UNSUPPORTED
    msg = L.attn_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg


def test_noalloc_decode_validates_like_the_workspace_decode():
    assert _decode_noalloc(maxq=5) == UNSUPPORTED
    assert "prefill" in L.attn_last_error().decode()
    assert _decode_noalloc(ks=NULL) == UNSUPPORTED
    assert _decode_noalloc(R=0) == OK
