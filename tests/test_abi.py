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
    assert names == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd", "fa_profile_events", "fa_status_string"]
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
