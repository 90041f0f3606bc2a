"""Dense fp64 form: scaled-dot-product attention written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (per batch b and query head h, with KV head g = h // (Hq/Hkv)):

    Sc   = scale * Q[b,h] K[b,g]^T                  (S x S)
    Sc[i, j] = -inf where j > i                      (only when causal)
    P    = row-softmax(Sc)
    O    = P V[b,g]
    L[i] = log sum_j exp(Sc[i, j])                   (natural log)

Sources: the attention formula and the inline causal mask in "Phase T14: 融合
Flash-Attention Kernel — Design Document" (section "什么是 flash-attention");
the statement that the flash method does not change this function, in
"FlashAttention 与 SDPA Backend" (section "先从 reference 语义出发"); GQA head
mapping kv_head = q_head / (Hq / Hkv) with contiguous groups, in "Phase 14:
Flash Attention 2 for SM120 — Design Document" (section "GQA 支持"); L as the
per-row logsumexp, in the T14 document (decision ②).

Backward: the plain chain rule through softmax, with no flash-specific
simplification.  For y = softmax(x) and upstream gradient g, dx = y * (g - <y, g>).
With dP = dO V^T:

    dS = P * (dP - rowsum(P * dP))
    dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO

and, for GQA, dK / dV of a KV head are the sums over the query heads that read
it (each query head's use of the shared K/V adds its own term).

Linear position bias (ALiBi, every function's ``alibi`` argument): a list of
one slope per query head, or None.  With slope a_h, the score of query i and
key j becomes scale * q_i . k_j - a_h * |i + offset - j| before the mask and
the softmax (offset = Skv - Sq, so the penalty is 0 on the bottom-right
diagonal and grows by a_h per key of distance).  "FlashAttention 与 SDPA
Backend" (section 失败场景与生产实现差距) lists ALiBi in its support matrix
without defining it; this form (and the slopes as an input) is a reading.  The
bias is a constant, so the gradients keep their form: dS = P * (dP - D).

Rows are processed in blocks only to bound memory; each row's softmax is always
taken over all of its unmasked columns at once.  Under a causal mask the columns
beyond the block's last row are all -inf and contribute exactly zero, so they
are not formed.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    return h // (Hq // Hkv)


def visible(rows, cols, causal, offset=0, window=None):
    """Boolean (len(rows), len(cols)) mask: key j visible to query i.

    causal: j <= i + offset, with offset = Skv - Sq (bottom-right alignment;
    0 when queries and keys have one length).  window (>= 0): also
    j >= i + offset - window.  Sources: the element mask of "Phase T14"
    (section 什么是 flash-attention) and "Phase 14" (section Causal Mask, which
    aligns a longer key sequence with kv_offset = kv_len - q_len).  The window
    is the sliding-window mask that "FlashAttention 与 SDPA Backend" lists in
    its support matrix; its left edge i + offset - window is a reading.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        vis &= j <= i + offset
    if window is not None:
        vis &= j >= i + offset - window
    return vis


def alibi_bias(rows, cols, slope, offset=0):
    """The linear position bias -slope * |i + offset - j| of queries ``rows`` (their
    positions) and keys ``cols``, shape (len(rows), len(cols))."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    return -float(slope) * np.abs(i + offset - j).astype(np.float64)


def _slope(alibi, h):
    return None if alibi is None else float(alibi[h])


def softmax_probs(q_rows, rows, k_head, scale, causal, offset=0, window=None, slope=None):
    """Rows of P and L for the query rows ``rows`` (their positions 0..Sq-1).

    q_rows: (n, D) query vectors of those rows; k_head: (Skv, D) keys of the
    KV head they read.  Returns (P, L, ncols) where P is (n, ncols): columns at
    or beyond ``ncols`` are all masked (causal) and so P is zero there.
    A row with no visible key gets P = 0 and L = -inf (its softmax is empty).
    ``slope``: the head's ALiBi slope, or None for no bias.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q_rows = _f64(q_rows)
    k_head = _f64(k_head)
    Skv = k_head.shape[0]
    ncols = min(Skv, int(rows.max()) + offset + 1) if causal else Skv
    ncols = max(ncols, 0)
    n = rows.shape[0]
    if ncols == 0:
        return np.zeros((n, 0)), np.full(n, -np.inf), 0
    sc = scale * (q_rows @ k_head[:ncols].T)
    if slope is not None:
        sc = sc + alibi_bias(rows, np.arange(ncols), slope, offset)
    vis = visible(rows, np.arange(ncols), causal, offset, window)
    sc = np.where(vis, sc, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, sc.max(axis=1), 0.0)[:, None]
    e = np.exp(sc - m)
    z = e.sum(axis=1, keepdims=True)
    P = np.where(any_vis[:, None], e / np.where(z > 0, z, 1.0), 0.0)
    with np.errstate(divide="ignore"):
        L = np.where(any_vis, (m + np.log(np.where(z > 0, z, 1.0)))[:, 0], -np.inf)
    return P, L, ncols


def _check_shapes(q, k, v):
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("q is [B,Hq,Sq,D]; k and v must be [B,Hkv,Skv,D]")
    Hkv, Skv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Sq, Skv, D


def sdpa_forward(q, k, v, scale, causal, heads=None, row_block=512, window=None, alibi=None):
    """O [B,Hq,Sq,D] and L [B,Hq,Sq] in fp64 (keys may be longer or shorter: Skv).

    ``heads``: optional list of (b, h) to compute; other heads are left NaN.
    ``window``: optional left window (see ``visible``).  ``alibi``: per-head
    slopes (see the module docstring) or None.
    """
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    off = Skv - Sq
    O = np.full((B, Hq, Sq, D), np.nan)
    L = np.full((B, Hq, Sq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = _kv_head(h, Hq, Hkv)
        kh, vh = _f64(k[b, g]), _f64(v[b, g])
        for r0 in range(0, Sq, row_block):
            r1 = min(Sq, r0 + row_block)
            rows = np.arange(r0, r1)
            P, Lr, nc = softmax_probs(q[b, h, r0:r1], rows, kh, scale, causal, off, window, _slope(alibi, h))
            O[b, h, r0:r1] = P @ vh[:nc]
            L[b, h, r0:r1] = Lr
    return O, L


def sdpa_forward_rows(q, k, v, scale, causal, b, h, rows, window=None, alibi=None):
    """O and L of selected rows of one (b, h): ((n, D), (n,)) in fp64."""
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    P, Lr, nc = softmax_probs(q[b, h][rows], rows, k[b, g], scale, causal, Skv - Sq, window, _slope(alibi, h))
    return P @ _f64(v[b, g][:nc]), Lr


def _row_block_backward(q_blk, rows, do_blk, kh, vh, scale, causal, off=0, window=None, slope=None):
    P, Lr, nc = softmax_probs(q_blk, rows, kh, scale, causal, off, window, slope)
    do_blk = _f64(do_blk)
    O = P @ vh[:nc]
    dP = do_blk @ vh[:nc].T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return P, Lr, nc, O, dS


def sdpa_backward(q, k, v, do, scale, causal, groups=None, row_block=512, window=None, alibi=None):
    """Gradients of sum(dO * O) with respect to q, k, v (fp64), plus O and L.

    ``groups``: optional list of (b, g) KV heads to compute; the query heads
    reading them are computed in full and everything else is left NaN.
    Keys may be longer or shorter than queries (Skv); ``window`` as in
    ``visible``; ``alibi`` per-head slopes or None.  Returns a dict with keys
    o, lse, dq, dk, dv.
    """
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    off = Skv - Sq
    G = Hq // Hkv
    out = {
        "o": np.full((B, Hq, Sq, D), np.nan),
        "lse": np.full((B, Hq, Sq), np.nan),
        "dq": np.full((B, Hq, Sq, D), np.nan),
        "dk": np.full((B, Hkv, Skv, D), np.nan),
        "dv": np.full((B, Hkv, Skv, D), np.nan),
    }
    todo = groups if groups is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        kh, vh = _f64(k[b, g]), _f64(v[b, g])
        dk = np.zeros((Skv, D))
        dv = np.zeros((Skv, D))
        for h in range(g * G, (g + 1) * G):
            qh = _f64(q[b, h])
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                rows = np.arange(r0, r1)
                P, Lr, nc, O, dS = _row_block_backward(
                    qh[r0:r1], rows, do[b, h, r0:r1], kh, vh, scale, causal, off, window, _slope(alibi, h))
                out["o"][b, h, r0:r1] = O
                out["lse"][b, h, r0:r1] = Lr
                out["dq"][b, h, r0:r1] = scale * (dS @ kh[:nc])
                dk[:nc] += scale * (dS.T @ qh[r0:r1])
                dv[:nc] += P.T @ _f64(do[b, h, r0:r1])
        out["dk"][b, g] = dk
        out["dv"][b, g] = dv
    return out


def sdpa_dq_rows(q, k, v, do, scale, causal, b, h, rows, window=None, alibi=None):
    """dQ of selected rows of one (b, h), (n, D) in fp64 (each row needs only its own P and dP)."""
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    kh, vh = _f64(k[b, g]), _f64(v[b, g])
    _, _, nc, _, dS = _row_block_backward(q[b, h][rows], rows, do[b, h][rows], kh, vh, scale, causal,
                                          Skv - Sq, window, _slope(alibi, h))
    return scale * (dS @ kh[:nc])


def sdpa_dkdv_keys(q, k, v, do, scale, causal, b, g, keys, window=None, alibi=None):
    """dK and dV of selected keys of one (b, KV head g): ((n, D), (n, D)) in fp64.

    A key's gradients are sums over the query rows that see it, of every query
    head of the group (the chain rule through the GQA mapping), so only those
    rows are formed: each one's full softmax row (its normalisation needs every
    key it sees), its dP row and its D, as in ``sdpa_backward``."""
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    off = Skv - Sq
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    kh, vh = _f64(k[b, g]), _f64(v[b, g])
    every = np.arange(Sq, dtype=np.int64)
    rows = every[visible(every, keys, causal, off, window).any(axis=1)]
    dk = np.zeros((keys.size, D))
    dv = np.zeros((keys.size, D))
    if rows.size == 0:
        return dk, dv
    for h in range(g * G, (g + 1) * G):
        qr, dor = _f64(q[b, h][rows]), _f64(do[b, h][rows])
        P, _, nc, _, dS = _row_block_backward(qr, rows, dor, kh, vh, scale, causal, off, window, _slope(alibi, h))
        inside = keys < nc  # keys past the rows' last visible column get nothing
        dk[inside] += scale * (dS[:, keys[inside]].T @ qr)
        dv[inside] += P[:, keys[inside]].T @ dor
    return dk, dv


def _seq_slices(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def sdpa_forward_varlen(q, k, v, cu_q, cu_k, scale, causal, window=None, alibi=None):
    """Packed variable-length batch: q [Hq, Tq, D], k, v [Hkv, Tk, D]; sequence b owns
    query rows cu_q[b]:cu_q[b+1] and keys cu_k[b]:cu_k[b+1] and is attended on its
    own (its offset is its own key length minus its own query length).
    Returns O [Hq, Tq, D], L [Hq, Tq]."""
    Hq, Tq, D = q.shape
    O = np.zeros((Hq, Tq, D))
    L = np.full((Hq, Tq), np.nan)
    for (q0, q1), (k0, k1) in zip(_seq_slices(cu_q), _seq_slices(cu_k)):
        if q1 == q0:
            continue
        Ob, Lb = sdpa_forward(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], scale, causal,
                              window=window, alibi=alibi)
        O[:, q0:q1], L[:, q0:q1] = Ob[0], Lb[0]
    return O, L


def sdpa_backward_varlen(q, k, v, do, cu_q, cu_k, scale, causal, window=None, alibi=None):
    """Packed variable-length backward (layouts as ``sdpa_forward_varlen``); dict o, lse, dq, dk, dv."""
    out = {"o": np.zeros(q.shape), "lse": np.full(q.shape[:2], np.nan), "dq": np.zeros(q.shape),
           "dk": np.zeros(k.shape), "dv": np.zeros(v.shape)}
    for (q0, q1), (k0, k1) in zip(_seq_slices(cu_q), _seq_slices(cu_k)):
        if q1 == q0:
            continue
        g = sdpa_backward(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], do[None, :, q0:q1],
                          scale, causal, window=window, alibi=alibi)
        out["o"][:, q0:q1], out["lse"][:, q0:q1], out["dq"][:, q0:q1] = g["o"][0], g["lse"][0], g["dq"][0]
        out["dk"][:, k0:k1], out["dv"][:, k0:k1] = g["dk"][0], g["dv"][0]
    return out
