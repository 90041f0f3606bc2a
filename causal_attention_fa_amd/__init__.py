"""Python binding of libfa.so, the MI355X fused causal attention library.

The functions ``fa_fwd``, ``fa_bwd``, ``fa_bwd_workspace_bytes`` and
``fa_status_string`` mirror the C ABI in ``include/fa.h`` one to one: they take
raw device addresses (ints) and sizes and return the C status code.  Every step
of the computation runs in the HIP kernels behind that ABI; this module only
marshals arguments.

``forward`` / ``backward`` are conveniences for PyTorch callers: they allocate
the outputs (and the backward workspace) with torch on the inputs' device, pass
torch's current stream, and raise ``FAError`` on a non-OK status.

There is no fallback: if libfa.so has not been built, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
    "FA_F32", "FA_F16", "FA_BF16", "FAError", "library_path", "lib",
    "fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "fa_profile_events",
    "forward", "backward",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_F32, FA_F16, FA_BF16 = range(3)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libfa.so")
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fa_status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(
                f"{library_path} is missing: build it first (python -m causal_attention_fa_amd.build)")
        L = ctypes.CDLL(library_path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_fwd.restype = i
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
        L.fa_bwd.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_profile_events.argtypes = [vp, i]
        L.fa_profile_events.restype = None
        _lib = L
    return _lib


# ------------------------------------------------------------------ raw C ABI

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal, dtype, stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, int(causal), dtype, stream)


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, causal, dtype,
           workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, int(causal), dtype,
                        workspace, workspace_bytes, stream)


def fa_bwd_workspace_bytes(B, Hq, Hkv, S, D) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def fa_profile_events(events, n) -> None:
    """events: address of an array of n hipEvent_t handles (or None to stop recording)."""
    lib().fa_profile_events(events, n)


# ------------------------------------------------------------------ torch conveniences

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q is [B,Hq,S,D]; k and v are [B,Hkv,S,D]")
    B, Hq, S, D = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError("q, k, v disagree on B, S or D")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    return B, Hq, k.shape[1], S, D


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


def forward(q, k, v, scale=None, causal=True, with_lse=True):
    """(o, lse) for device tensors q [B,Hq,S,D], k, v [B,Hkv,S,D]; lse is fp32 [B,Hq,S] or None."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if with_lse else None
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr() if with_lse else None,
                B, Hq, Hkv, S, D, scale, causal, _dtype_code(q), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, lse


def backward(q, k, v, o, lse, do, scale=None, causal=True, workspace=None):
    """(dq, dk, dv) for the forward's inputs, its outputs o and lse, and dO."""
    torch = _torch()
    B, Hq, Hkv, S, D = _check(q, k, v)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("o and dO must match q")
    if lse.shape != (B, Hq, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B,Hq,S]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = fa_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, S, D, scale, causal,
                _dtype_code(q), workspace.data_ptr(), workspace.numel(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv
