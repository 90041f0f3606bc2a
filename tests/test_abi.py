"""The C-ABI library: loads, exports what include/fa.h declares, and rejects bad
arguments on the host before touching the GPU (CPU only; no kernel launches).

Every call here either fails argument checking or is an empty problem, both of
which return before any HIP call.
"""
import math
import os
import re

import pytest

import causal_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000  # a 16-byte aligned fake address: never dereferenced by these calls


def declared_functions():
    with open(os.path.join(ROOT, "include", "fa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["fa_bwd", "fa_bwd_ex", "fa_bwd_ex_workspace_bytes", "fa_bwd_noalloc", "fa_bwd_workspace_bytes",
                     "fa_fwd",
                     "fa_fwd_ex", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_profile_events",
                     "fa_status_string"]
    L = fa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert fa.fa_status_string(fa.FA_OK) == "FA_OK"
    assert fa.fa_status_string(fa.FA_ERR_INVALID_ARG) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(fa.FA_ERR_UNSUPPORTED) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(fa.FA_ERR_WORKSPACE) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_string(fa.FA_ERR_HIP) == "FA_ERR_HIP"
    assert fa.fa_status_string(99) == "FA_ERR_UNKNOWN"


def test_workspace_bytes():
    n = fa.fa_bwd_workspace_bytes(1, 32, 8, 16384, 128)
    assert n == 32 * 16384 * 4 and n % 256 == 0
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 3, 64) == 256
    assert fa.fa_bwd_workspace_bytes(0, 2, 2, 3, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 3, 2, 8, 64) == 0      # rejected shape
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 8, 96) == 0      # unsupported D


def fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=4, Hkv=2, S=16, D=64, scale=0.125, causal=1,
                dtype=fa.FA_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


def bwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, dO=A, dq=A, dk=A, dv=A, B=1, Hq=4, Hkv=2, S=16, D=64,
                scale=0.125, causal=1, dtype=fa.FA_BF16, workspace=A,
                workspace_bytes=fa.fa_bwd_workspace_bytes(1, 4, 2, 16, 64), stream=None)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("call", [fwd, bwd])
@pytest.mark.parametrize("kw,expect", [
    ({"q": None}, fa.FA_ERR_INVALID_ARG),
    ({"k": None}, fa.FA_ERR_INVALID_ARG),
    ({"v": None}, fa.FA_ERR_INVALID_ARG),
    ({"q": A + 8}, fa.FA_ERR_INVALID_ARG),
    ({"v": A + 2}, fa.FA_ERR_INVALID_ARG),
    ({"Hq": 3}, fa.FA_ERR_INVALID_ARG),
    ({"Hkv": 0}, fa.FA_ERR_INVALID_ARG),
    ({"B": -1}, fa.FA_ERR_INVALID_ARG),
    ({"S": -5}, fa.FA_ERR_INVALID_ARG),
    ({"D": -64}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 7}, fa.FA_ERR_INVALID_ARG),
    ({"scale": math.nan}, fa.FA_ERR_INVALID_ARG),
    ({"scale": math.inf}, fa.FA_ERR_INVALID_ARG),
    ({"D": 96}, fa.FA_ERR_UNSUPPORTED),
    ({"D": 256}, fa.FA_ERR_UNSUPPORTED),
    ({"D": 0}, fa.FA_ERR_UNSUPPORTED),
    ({"scale": 0.0}, fa.FA_ERR_UNSUPPORTED),
    ({"scale": -0.125}, fa.FA_ERR_UNSUPPORTED),
    ({"B": 0}, fa.FA_OK),
    ({"S": 0}, fa.FA_OK),
    ({"B": 0, "q": None, "o": None}, fa.FA_OK),
    ({"S": 0, "Hq": 3}, fa.FA_ERR_INVALID_ARG),
])
def test_argument_checks(call, kw, expect):
    assert call(**kw) == expect


@pytest.mark.parametrize("kw", [{"o": None}, {"o": A + 4}, {"lse": A + 4}])
def test_forward_output_checks(kw):
    assert fwd(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,expect", [
    ({"lse": None}, fa.FA_ERR_INVALID_ARG),
    ({"dO": None}, fa.FA_ERR_INVALID_ARG),
    ({"dq": None}, fa.FA_ERR_INVALID_ARG),
    ({"dk": A + 8}, fa.FA_ERR_INVALID_ARG),
    ({"dv": None}, fa.FA_ERR_INVALID_ARG),
    ({"workspace": None}, fa.FA_ERR_INVALID_ARG),
    ({"workspace": A + 4}, fa.FA_ERR_INVALID_ARG),
    ({"workspace_bytes": 255}, fa.FA_ERR_WORKSPACE),
    ({"workspace_bytes": 0}, fa.FA_ERR_WORKSPACE),
])
def test_backward_checks(kw, expect):
    assert bwd(**kw) == expect


def test_profile_events_toggle_without_gpu():
    fa.fa_profile_events(None, 0)      # off: pure host state, no HIP call


def test_python_wrappers_need_device_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


# ------------------------------------------------------------------ extended problems

def test_params_struct_layout():
    import ctypes
    P = fa.fa_params_t
    # int B,Hq,Hkv,Sq,Skv,D; float scale; int causal, window; two pointers; int total_q, total_k; enum dtype;
    # a pointer (after 4 bytes of padding)
    assert P.scale.offset == 24 and P.window.offset == 32
    assert P.cu_seqlens_q.offset == 40 and P.cu_seqlens_k.offset == 48
    assert P.total_q.offset == 56 and P.dtype.offset == 64
    assert P.alibi_slopes.offset == 72 and ctypes.sizeof(P) == 80


def ex_params(**kw):
    base = dict(B=1, Hq=4, Hkv=2, Sq=16, Skv=24, D=64, scale=0.125, causal=True, window=None,
                dtype=fa.FA_BF16)
    base.update(kw)
    return fa.params(**base)


def fwd_ex(p=None, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, stream=None)
    args.update(kw)
    return fa.fa_fwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"],
                        ex_params() if p is None else p, args["stream"])


def bwd_ex(p=None, **kw):
    p = ex_params() if p is None else p
    args = dict(q=A, k=A, v=A, o=A, lse=A, dO=A, dq=A, dk=A, dv=A, workspace=A,
                workspace_bytes=fa.fa_bwd_ex_workspace_bytes(p), stream=None)
    args.update(kw)
    return fa.fa_bwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dO"], args["dq"],
                        args["dk"], args["dv"], p, args["workspace"], args["workspace_bytes"], args["stream"])


def test_ex_null_params():
    assert fa.lib().fa_fwd_ex(A, A, A, A, A, None, None) == fa.FA_ERR_INVALID_ARG
    assert fa.lib().fa_bwd_ex(A, A, A, A, A, A, A, A, A, None, A, 1 << 20, None) == fa.FA_ERR_INVALID_ARG
    assert fa.lib().fa_bwd_ex_workspace_bytes(None) == 0


@pytest.mark.parametrize("call", [fwd_ex, bwd_ex])
@pytest.mark.parametrize("pk,expect", [
    ({"Sq": -1}, fa.FA_ERR_INVALID_ARG),
    ({"Skv": -1}, fa.FA_ERR_INVALID_ARG),
    ({"Hq": 3}, fa.FA_ERR_INVALID_ARG),
    ({"Hq": 0}, fa.FA_ERR_INVALID_ARG),          # key rows but no query head
    ({"B": 0}, fa.FA_OK),
    ({"Sq": 0, "Skv": 0}, fa.FA_OK),
    ({"D": 96}, fa.FA_ERR_UNSUPPORTED),
    ({"scale": 0.0}, fa.FA_ERR_UNSUPPORTED),
    ({"scale": math.nan}, fa.FA_ERR_INVALID_ARG),
    ({"dtype": 5}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_q": A}, fa.FA_ERR_INVALID_ARG),                       # only one offset array
    ({"cu_seqlens_k": A}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_q": A + 2, "cu_seqlens_k": A, "total_q": 4, "total_k": 4}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_q": A, "cu_seqlens_k": A, "total_q": -1, "total_k": 4}, fa.FA_ERR_INVALID_ARG),
    ({"cu_seqlens_q": A, "cu_seqlens_k": A, "total_q": 0, "total_k": 0}, fa.FA_OK),
    ({"Sq": (1 << 29) + 1}, fa.FA_ERR_UNSUPPORTED),
    ({"Skv": (1 << 29) + 1}, fa.FA_ERR_UNSUPPORTED),
    ({"B": 1 << 20, "Hq": 1 << 10, "Hkv": 1 << 10, "Sq": 1 << 10, "Skv": 16}, fa.FA_ERR_UNSUPPORTED),
])
def test_ex_argument_checks(call, pk, expect):
    assert call(ex_params(**pk)) == expect


def test_ex_forward_empty_sides():
    # no query rows: nothing to compute, no pointer is needed
    assert fwd_ex(ex_params(Sq=0), q=None, k=None, v=None, o=None, lse=None) == fa.FA_OK
    # query rows need q and o
    assert fwd_ex(q=None) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(o=A + 4) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(lse=A + 4) == fa.FA_ERR_INVALID_ARG
    # key rows need k and v
    assert fwd_ex(k=None) == fa.FA_ERR_INVALID_ARG
    assert fwd_ex(v=A + 8) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [{"lse": None}, {"dO": None}, {"dq": A + 8}, {"dk": None}, {"dv": A + 4},
                                {"q": None}, {"k": None}])
def test_ex_backward_pointer_checks(kw):
    assert bwd_ex(**kw) == fa.FA_ERR_INVALID_ARG


def test_ex_backward_workspace():
    p = ex_params()
    n = fa.fa_bwd_ex_workspace_bytes(p)
    assert n == 256                                      # 4 heads x 16 rows x 4 bytes, rounded up
    assert bwd_ex(p, workspace_bytes=n - 1) == fa.FA_ERR_WORKSPACE
    assert bwd_ex(p, workspace=None) == fa.FA_ERR_INVALID_ARG
    big = ex_params(Hq=32, Hkv=8, Sq=16384, Skv=16384, D=128)
    assert fa.fa_bwd_ex_workspace_bytes(big) == 32 * 16384 * 4
    packed = ex_params(cu_seqlens_q=A, cu_seqlens_k=A, total_q=1000, total_k=3000, B=5)
    assert fa.fa_bwd_ex_workspace_bytes(packed) == 16128   # heads x total query rows x 4 bytes, to 256
    assert fa.fa_bwd_ex_workspace_bytes(ex_params(Hq=3)) == 0


def test_ex_backward_without_queries_needs_no_query_buffers():
    # keys but no queries: dk and dv are still written (zeros), so only the key-side buffers are needed,
    # but that is a launch: the empty-problem form (no rows at all) is the only pure host case here
    p = ex_params(Sq=0, Skv=0)
    assert bwd_ex(p, q=None, k=None, v=None, o=None, lse=None, dO=None, dq=None, dk=None, dv=None,
                  workspace=None) == fa.FA_OK
    p = ex_params(Sq=0)
    assert fa.fa_bwd_ex_workspace_bytes(p) == 0
    assert bwd_ex(p, dk=None) == fa.FA_ERR_INVALID_ARG     # key rows need dk, checked before any launch


# ------------------------------------------------------------------ split-KV decode

def splitkv(p=None, num_splits=0, **kw):
    p = ex_params(Sq=1, Skv=4096) if p is None else p
    args = dict(q=A, k=A, v=A, o=A, lse=A, workspace=A, workspace_bytes=fa.fa_fwd_splitkv_workspace_bytes(p, num_splits),
                stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv(args["q"], args["k"], args["v"], args["o"], args["lse"], p, num_splits,
                             args["workspace"], args["workspace_bytes"], args["stream"])


def test_splitkv_workspace_sizing():
    # 1 x 4 query heads x 1 row, 4096 keys in 128-key tiles: the library picks
    # min(512 / (B*Hkv), tiles / 2) = 16 ranges; each holds rows x (D + 1) floats
    p = ex_params(Sq=1, Skv=4096)
    assert fa.fa_fwd_splitkv_workspace_bytes(p, 0) == 16 * 4 * 65 * 4
    assert fa.fa_fwd_splitkv_workspace_bytes(p, 3) == 3328     # 3 x 4 x 65 x 4 = 3120, to 256
    assert fa.fa_fwd_splitkv_workspace_bytes(p, 10 ** 6) == fa.fa_fwd_splitkv_workspace_bytes(p, 32)  # one per tile
    f32 = ex_params(Sq=1, Skv=4096, dtype=fa.FA_F32)  # 64-key tiles
    assert fa.fa_fwd_splitkv_workspace_bytes(f32, 10 ** 6) == 64 * 4 * 65 * 4
    assert fa.fa_fwd_splitkv_workspace_bytes(ex_params(Sq=17, Skv=100), 0) == 0   # 2 x 17 > 32 rows
    assert fa.fa_fwd_splitkv_workspace_bytes(ex_params(Sq=0), 0) == 0


@pytest.mark.parametrize("kw,expect", [
    ({"workspace": None}, fa.FA_ERR_INVALID_ARG),
    ({"workspace": A + 8}, fa.FA_ERR_INVALID_ARG),
    ({"workspace_bytes": 100}, fa.FA_ERR_WORKSPACE),
    ({"q": None}, fa.FA_ERR_INVALID_ARG),
    ({"o": A + 4}, fa.FA_ERR_INVALID_ARG),
    ({"k": None}, fa.FA_ERR_INVALID_ARG),
    ({"lse": A + 4}, fa.FA_ERR_INVALID_ARG),
])
def test_splitkv_checks(kw, expect):
    assert splitkv(**kw) == expect


def test_splitkv_shape_limits():
    # group rows beyond one 32-column block
    assert splitkv(ex_params(Hq=8, Hkv=2, Sq=9, Skv=100), workspace_bytes=1 << 20) == fa.FA_ERR_UNSUPPORTED
    # no query rows: a no-op that needs no buffers
    assert splitkv(ex_params(Sq=0), q=None, k=None, v=None, o=None, lse=None, workspace=None) == fa.FA_OK
    assert splitkv(ex_params(D=96, Sq=1)) == fa.FA_ERR_UNSUPPORTED


def test_noalloc_backward_host_checks():
    """fa_bwd_noalloc checks its arguments like fa_bwd, and rejects a problem with more
    query rows than its static array holds, all before any HIP call."""
    call = lambda **kw: fa.fa_bwd_noalloc(**dict(dict(
        q=A, k=A, v=A, o=A, lse=A, dO=A, dq=A, dk=A, dv=A, B=1, Hq=4, Hkv=2, S=16, D=64, scale=0.125, causal=1,
        dtype=fa.FA_BF16, stream=None), **kw))
    assert call(q=None) == fa.FA_ERR_INVALID_ARG
    assert call(dv=A + 4) == fa.FA_ERR_INVALID_ARG
    assert call(Hq=3) == fa.FA_ERR_INVALID_ARG
    assert call(D=96) == fa.FA_ERR_UNSUPPORTED
    assert call(B=0) == fa.FA_OK                          # empty: a no-op
    rows = fa.FA_BWD_NOALLOC_MAX_ROWS
    assert call(Hq=64, Hkv=64, S=rows // 64 + 1) == fa.FA_ERR_WORKSPACE


def test_alibi_host_checks():
    """Slopes must be 4-byte aligned; the split-KV path has no position bias."""
    assert fwd_ex(ex_params(alibi_slopes=A + 2)) == fa.FA_ERR_INVALID_ARG
    assert bwd_ex(ex_params(alibi_slopes=A + 2)) == fa.FA_ERR_INVALID_ARG
    p = ex_params(Sq=1, Skv=64, alibi_slopes=A)
    assert fa.fa_fwd_splitkv_workspace_bytes(p, 0) == 0
    assert fa.fa_fwd_splitkv(A, A, A, A, A, p, 0, A, 1 << 20, None) == fa.FA_ERR_UNSUPPORTED
    # an empty problem with slopes is still a no-op
    assert fwd_ex(ex_params(B=0, alibi_slopes=A)) == fa.FA_OK
