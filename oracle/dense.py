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


def softmax_probs(q_rows, rows, k_head, scale, causal):
    """Rows of P and L for the query rows ``rows`` (their positions 0..S-1).

    q_rows: (n, D) query vectors of those rows; k_head: (S, D) keys of the
    KV head they read.  Returns (P, L, ncols) where P is (n, ncols): columns at
    or beyond ``ncols`` are all masked (causal) and so P is zero there.
    """
    rows = np.asarray(rows, dtype=np.int64)
    q_rows = _f64(q_rows)
    k_head = _f64(k_head)
    S = k_head.shape[0]
    ncols = int(rows.max()) + 1 if causal else S
    sc = scale * (q_rows @ k_head[:ncols].T)
    if causal:
        sc = np.where(np.arange(ncols)[None, :] > rows[:, None], -np.inf, sc)
    m = sc.max(axis=1, keepdims=True)
    e = np.exp(sc - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0], ncols


def _check_shapes(q, k, v):
    B, Hq, S, D = q.shape
    if k.shape[0] != B or k.shape[2:] != (S, D) or v.shape != k.shape:
        raise ValueError("q is [B,Hq,S,D]; k and v must be [B,Hkv,S,D]")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, S, D


def sdpa_forward(q, k, v, scale, causal, heads=None, row_block=512):
    """O [B,Hq,S,D] and L [B,Hq,S] in fp64.

    ``heads``: optional list of (b, h) to compute; other heads are left NaN.
    """
    B, Hq, Hkv, S, D = _check_shapes(q, k, v)
    O = np.full((B, Hq, S, D), np.nan)
    L = np.full((B, Hq, S), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = _kv_head(h, Hq, Hkv)
        kh, vh = _f64(k[b, g]), _f64(v[b, g])
        for r0 in range(0, S, row_block):
            r1 = min(S, r0 + row_block)
            rows = np.arange(r0, r1)
            P, Lr, nc = softmax_probs(q[b, h, r0:r1], rows, kh, scale, causal)
            O[b, h, r0:r1] = P @ vh[:nc]
            L[b, h, r0:r1] = Lr
    return O, L


def sdpa_forward_rows(q, k, v, scale, causal, b, h, rows):
    """O and L of selected rows of one (b, h): ((n, D), (n,)) in fp64."""
    B, Hq, Hkv, S, D = _check_shapes(q, k, v)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    P, Lr, nc = softmax_probs(q[b, h][rows], rows, k[b, g], scale, causal)
    return P @ _f64(v[b, g][:nc]), Lr


def _row_block_backward(q_blk, rows, do_blk, kh, vh, scale, causal):
    P, Lr, nc = softmax_probs(q_blk, rows, kh, scale, causal)
    do_blk = _f64(do_blk)
    O = P @ vh[:nc]
    dP = do_blk @ vh[:nc].T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return P, Lr, nc, O, dS


def sdpa_backward(q, k, v, do, scale, causal, groups=None, row_block=512):
    """Gradients of sum(dO * O) with respect to q, k, v (fp64), plus O and L.

    ``groups``: optional list of (b, g) KV heads to compute; the query heads
    reading them are computed in full and everything else is left NaN.
    Returns a dict with keys o, lse, dq, dk, dv.
    """
    B, Hq, Hkv, S, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    out = {
        "o": np.full((B, Hq, S, D), np.nan),
        "lse": np.full((B, Hq, S), np.nan),
        "dq": np.full((B, Hq, S, D), np.nan),
        "dk": np.full((B, Hkv, S, D), np.nan),
        "dv": np.full((B, Hkv, S, D), np.nan),
    }
    todo = groups if groups is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        kh, vh = _f64(k[b, g]), _f64(v[b, g])
        dk = np.zeros((S, D))
        dv = np.zeros((S, D))
        for h in range(g * G, (g + 1) * G):
            qh = _f64(q[b, h])
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                rows = np.arange(r0, r1)
                P, Lr, nc, O, dS = _row_block_backward(
                    qh[r0:r1], rows, do[b, h, r0:r1], kh, vh, scale, causal)
                out["o"][b, h, r0:r1] = O
                out["lse"][b, h, r0:r1] = Lr
                out["dq"][b, h, r0:r1] = scale * (dS @ kh[:nc])
                dk[:nc] += scale * (dS.T @ qh[r0:r1])
                dv[:nc] += P.T @ _f64(do[b, h, r0:r1])
        out["dk"][b, g] = dk
        out["dv"][b, g] = dv
    return out


def sdpa_dq_rows(q, k, v, do, scale, causal, b, h, rows):
    """dQ of selected rows of one (b, h), (n, D) in fp64 (each row needs only its own P and dP)."""
    B, Hq, Hkv, S, D = _check_shapes(q, k, v)
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    kh, vh = _f64(k[b, g]), _f64(v[b, g])
    _, _, nc, _, dS = _row_block_backward(q[b, h][rows], rows, do[b, h][rows], kh, vh, scale, causal)
    return scale * (dS @ kh[:nc])
