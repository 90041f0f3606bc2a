"""Python binding of libfa.so, the MI355X fused causal attention library.

The functions ``fa_fwd``, ``fa_bwd``, ``fa_bwd_noalloc``, ``fa_bwd_workspace_bytes``, ``fa_fwd_ex``,
``fa_bwd_ex``, ``fa_bwd_ex_workspace_bytes`` and ``fa_status_string`` mirror
the C ABI in ``include/fa.h`` one to one: they take raw device addresses (ints)
and sizes (or an ``fa_params_t``) and return the C status code.  Every step of
the computation runs in the HIP kernels behind that ABI; this module only
marshals arguments.

``forward`` / ``backward`` (dense batches, queries and keys of any lengths,
optional sliding window) and ``forward_varlen`` / ``backward_varlen`` (packed
variable-length batches) are conveniences for PyTorch callers: they allocate
the outputs (and the backward workspace) with torch on the inputs' device, pass
torch's current stream, and raise ``FAError`` on a non-OK status.
``attention`` wraps ``forward`` and ``backward`` as one differentiable torch
operation: its autograd node keeps the forward's O and L for the backward.

There is no fallback: if libfa.so has not been built, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
    "FA_F32", "FA_F16", "FA_BF16", "FAError", "library_path", "lib",
    "fa_fwd", "fa_bwd", "fa_bwd_noalloc", "FA_BWD_NOALLOC_MAX_ROWS", "fa_bwd_workspace_bytes",
    "fa_status_string", "fa_profile_events",
    "fa_params_t", "params", "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_ex_workspace_bytes",
    "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes",
    "forward", "backward", "forward_varlen", "backward_varlen", "forward_splitkv", "attention",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_F32, FA_F16, FA_BF16 = range(3)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libfa.so")
_lib = None


class fa_params_t(ctypes.Structure):
    """The C struct fa_params_t (include/fa.h), field for field."""
    _fields_ = [
        ("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
        ("Sq", ctypes.c_int), ("Skv", ctypes.c_int), ("D", ctypes.c_int),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("window", ctypes.c_int),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int), ("total_k", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("alibi_slopes", ctypes.c_void_p),
    ]


def params(B, Hq, Hkv, Sq, Skv, D, scale, causal=True, window=None, dtype=FA_BF16,
           cu_seqlens_q=None, cu_seqlens_k=None, total_q=0, total_k=0, alibi_slopes=None) -> fa_params_t:
    """An fa_params_t; ``window=None`` means no window, cu_seqlens_* and alibi_slopes
    (Hq fp32 slopes) are device addresses."""
    return fa_params_t(B, Hq, Hkv, Sq, Skv, D, scale, int(causal), -1 if window is None else int(window),
                       cu_seqlens_q, cu_seqlens_k, total_q, total_k, dtype, alibi_slopes)


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
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa_bwd_noalloc.restype = i
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_profile_events.argtypes = [vp, i]
        L.fa_profile_events.restype = None
        pp = ctypes.POINTER(fa_params_t)
        L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, pp, vp]
        L.fa_fwd_ex.restype = i
        L.fa_bwd_ex_workspace_bytes.argtypes = [pp]
        L.fa_bwd_ex_workspace_bytes.restype = sz
        L.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, sz, vp]
        L.fa_bwd_ex.restype = i
        L.fa_fwd_splitkv_workspace_bytes.argtypes = [pp, i]
        L.fa_fwd_splitkv_workspace_bytes.restype = sz
        L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, pp, i, vp, sz, vp]
        L.fa_fwd_splitkv.restype = i
        _lib = L
    return _lib


# ------------------------------------------------------------------ raw C ABI

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal, dtype, stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, scale, int(causal), dtype, stream)


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, causal, dtype,
           workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, int(causal), dtype,
                        workspace, workspace_bytes, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, causal, dtype, stream) -> int:
    return lib().fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, D, scale, int(causal), dtype,
                                stream)


FA_BWD_NOALLOC_MAX_ROWS = 1 << 22


def fa_bwd_workspace_bytes(B, Hq, Hkv, S, D) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, Hq, Hkv, S, D))


def _pp(p):
    return None if p is None else ctypes.byref(p)


def fa_fwd_ex(q, k, v, o, lse, p, stream) -> int:
    """p: an fa_params_t (or None, which the library rejects)."""
    return lib().fa_fwd_ex(q, k, v, o, lse, _pp(p), stream)


def fa_bwd_ex_workspace_bytes(p) -> int:
    return int(lib().fa_bwd_ex_workspace_bytes(_pp(p)))


def fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, p, workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, _pp(p), workspace, workspace_bytes, stream)


def fa_fwd_splitkv_workspace_bytes(p, num_splits=0) -> int:
    return int(lib().fa_fwd_splitkv_workspace_bytes(_pp(p), num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, p, num_splits, workspace, workspace_bytes, stream) -> int:
    return lib().fa_fwd_splitkv(q, k, v, o, lse, _pp(p), num_splits, workspace, workspace_bytes, stream)


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


def _same(ts, what):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != ts[0].dtype:
            raise ValueError(f"{what} must be contiguous device tensors of one dtype")


def _check(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q is [B,Hq,Sq,D]; k and v are [B,Hkv,Skv,D]")
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q, k, v disagree on B or D")
    _same((q, k, v), "q, k, v")
    return B, Hq, k.shape[1], Sq, k.shape[2], D


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _slopes(alibi, Hq, device):
    """Address of a contiguous fp32 device vector of Hq ALiBi slopes, or None."""
    if alibi is None:
        return None
    torch = _torch()
    if (not isinstance(alibi, torch.Tensor) or alibi.dtype != torch.float32 or alibi.dim() != 1
            or alibi.numel() != Hq or not alibi.is_contiguous() or alibi.device != device):
        raise ValueError("alibi must be a contiguous fp32 vector of Hq slopes on the inputs' device")
    return alibi.data_ptr()


def forward(q, k, v, scale=None, causal=True, with_lse=True, window=None, alibi=None):
    """(o, lse) for device tensors q [B,Hq,Sq,D], k, v [B,Hkv,Skv,D]; lse is fp32 [B,Hq,Sq] or None.

    With Sq == Skv, no window and no bias this calls fa_fwd, otherwise fa_fwd_ex
    (causal diagonal aligned bottom-right; ``window`` keys before the diagonal
    stay visible; ``alibi`` an fp32 device vector of Hq slopes)."""
    torch = _torch()
    B, Hq, Hkv, Sq, Skv, D = _check(q, k, v)
    scale = _scale(scale, D)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if with_lse else None
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse))
    if Sq == Skv and window is None and alibi is None:
        st = fa_fwd(*ptrs, B, Hq, Hkv, Sq, D, scale, causal, _dtype_code(q), _stream(q))
    else:
        p = params(B, Hq, Hkv, Sq, Skv, D, scale, causal, window, _dtype_code(q),
                   alibi_slopes=_slopes(alibi, Hq, q.device))
        st = fa_fwd_ex(*ptrs, p, _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, lse


def _workspace(nbytes, workspace, device):
    if workspace is None:
        workspace = _torch().empty(max(nbytes, 256), dtype=_torch().uint8, device=device)
    return workspace


def backward(q, k, v, o, lse, do, scale=None, causal=True, workspace=None, window=None, alibi=None):
    """(dq, dk, dv) for the forward's inputs, its outputs o and lse, and dO."""
    torch = _torch()
    B, Hq, Hkv, Sq, Skv, D = _check(q, k, v)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("o and dO must match q")
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B,Hq,Sq]")
    scale = _scale(scale, D)
    dense = Sq == Skv and window is None and alibi is None
    p = params(B, Hq, Hkv, Sq, Skv, D, scale, causal, window, _dtype_code(q),
               alibi_slopes=_slopes(alibi, Hq, q.device))
    workspace = _workspace(fa_bwd_ex_workspace_bytes(p), workspace, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ptrs = tuple(_ptr(t) for t in (q, k, v, o, lse, do, dq, dk, dv))
    if dense:
        st = fa_bwd(*ptrs, B, Hq, Hkv, Sq, D, scale, causal, _dtype_code(q), workspace.data_ptr(),
                    workspace.numel(), _stream(q))
    else:
        st = fa_bwd_ex(*ptrs, p, workspace.data_ptr(), workspace.numel(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def _check_varlen(q, k, v, cu_q, cu_k):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q is [Hq,total_q,D]; k and v are [Hkv,total_k,D]")
    _same((q, k, v), "q, k, v")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_cuda or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 device vectors")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need B + 1 entries each")
    return cu_q.numel() - 1, q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2]


def _varlen_params(q, k, v, cu_q, cu_k, max_q, max_k, scale, causal, window, alibi=None):
    B, Hq, Hkv, Tq, Tk, D = _check_varlen(q, k, v, cu_q, cu_k)
    return params(B, Hq, Hkv, int(max_q), int(max_k), D, _scale(scale, D), causal, window, _dtype_code(q),
                  cu_q.data_ptr(), cu_k.data_ptr(), Tq, Tk, _slopes(alibi, Hq, q.device))


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None, causal=True,
                   window=None, alibi=None):
    """Packed batch: q [Hq,total_q,D], k, v [Hkv,total_k,D], cu_seqlens_* int32 [B+1] on the device.
    Returns o [Hq,total_q,D] and lse fp32 [Hq,total_q]; max_seqlen_* bound the per-sequence lengths."""
    torch = _torch()
    p = _varlen_params(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, window,
                       alibi)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    st = fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), p, _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_ex")
    return o, lse


def backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                    causal=True, window=None, workspace=None, alibi=None):
    """(dq, dk, dv) of a packed batch (layouts as ``forward_varlen``)."""
    torch = _torch()
    p = _varlen_params(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, window,
                       alibi)
    for t in (o, do):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("o and dO must match q")
    if lse.shape != q.shape[:2] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [Hq,total_q]")
    workspace = _workspace(fa_bwd_ex_workspace_bytes(p), workspace, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd_ex(*(_ptr(t) for t in (q, k, v, o, lse, do, dq, dk, dv)), p, workspace.data_ptr(),
                   workspace.numel(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_ex")
    return dq, dk, dv


def forward_splitkv(q, k, v, scale=None, causal=True, window=None, num_splits=0, cu_seqlens_q=None,
                    cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, workspace=None):
    """(o, lse) by the split-KV decode path (fa_fwd_splitkv).

    Dense: q [B,Hq,Sq,D], k, v [B,Hkv,Skv,D].  Packed: q [Hq,total_q,D], k, v
    [Hkv,total_k,D] with cu_seqlens_* and max_seqlen_* as in ``forward_varlen``.
    (Hq / Hkv) * Sq must be at most 32; ``num_splits`` <= 0 lets the library choose."""
    torch = _torch()
    if cu_seqlens_q is None:
        B, Hq, Hkv, Sq, Skv, D = _check(q, k, v)
        p = params(B, Hq, Hkv, Sq, Skv, D, _scale(scale, D), causal, window, _dtype_code(q))
        lse_shape = (B, Hq, Sq)
    else:
        p = _varlen_params(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, window)
        lse_shape = tuple(q.shape[:2])
    nbytes = fa_fwd_splitkv_workspace_bytes(p, num_splits)
    workspace = _workspace(nbytes, workspace, q.device)
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    st = fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), p, num_splits, workspace.data_ptr(),
                        workspace.numel(), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_splitkv")
    return o, lse


_attention_fn = None


def attention(q, k, v, scale=None, causal=True, window=None):
    """o for device tensors q [B,Hq,Sq,D], k, v [B,Hkv,Skv,D], differentiable in q, k and v.

    The forward runs ``forward`` and keeps its outputs o and L (the logsumexp, the only
    state the backward needs); the backward runs ``backward`` on them with the incoming
    dO.  Both passes are the library's kernels; this only connects them to autograd."""
    global _attention_fn
    if _attention_fn is None:
        torch = _torch()

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal, window):
                o, lse = forward(q, k, v, scale=scale, causal=causal, window=window)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.cfg = (scale, causal, window)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                scale, causal, window = ctx.cfg
                dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), scale=scale, causal=causal,
                                      window=window)
                return dq, dk, dv, None, None, None

        _attention_fn = _Attention
    return _attention_fn.apply(q, k, v, scale, causal, window)
