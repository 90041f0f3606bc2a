"""Tiled fp64 form: the flash method's own steps, in the pages' order and notation.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Forward (``online_forward``): Q-tile outer loop, KV-tile inner loop (the FA2
order of "Phase 14: Flash Attention 2 for SM120 — Design Document", section
"FA2 算法", and of the udemi.tech "Flash Attention" pseudocode).  Per query row
the state is the running max m, the running sum l and the unnormalised output
acc ("Phase T14: 融合 Flash-Attention Kernel — Design Document", section
"什么是 flash-attention"; "FlashAttention 与 SDPA Backend", section "Online
softmax 的三个状态").  For each KV tile with scores s:

    m_new = max(m, rowmax(s))
    p     = exp(s - m_new)            (0 where s is masked: the isfinite guard
                                       of the runnable reference on the SDPA page)
    l     = l * exp(m - m_new) + rowsum(p)
    acc   = acc * exp(m - m_new) + p V_tile
    m     = m_new
    ...   out = acc / l,  L = m + log(l)

A KV tile that lies wholly above the diagonal of the current Q tile is never
visited: the loop over KV tiles stops once the tile's first key is beyond the
Q tile's last row (tile-level causal skip of the Phase-14 document, section
"Causal Mask"; the ``break`` condition of the udemi pseudocode).  Inside a
visited tile, keys after the query row are -inf.  The last tile may be partial
(end = min(start + B, N)).

Where every score of a row in a tile is masked and m is still -inf, the
exponent's reference point is taken as 0 instead of -inf so that
exp(-inf - (-inf)) never appears (the pages' guard keeps p = 0 there).

Backward (``online_backward``): "Phase T14" section "什么是 flash-attention"
(the per-(i, j) recompute formulas) and decision ③.  First pass:
D[i] = sum_d dO[i, d] * O[i, d].  Then KV tiles outer, Q tiles inner (only
Q tiles with a row at or after the KV tile's first key when causal):

    s  = scale * Q_i K_j^T ;  p = exp(s - L[i])     (0 where masked)
    dV_j += p^T dO_i
    dp = dO_i V_j^T
    ds = p * (dp - D[i])
    dQ_i += scale * ds K_j ;  dK_j += scale * ds^T Q_i

GQA: the query heads of a group are visited inside the KV tile's loop, so dK/dV
of the shared KV head sum over the group (chain rule; the pages' GQA section
gives the forward mapping only).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _mask(s, q_pos, k_pos, causal, Skv, off=0, window=None):
    bad = k_pos[None, :] >= Skv
    if causal:
        bad = bad | (k_pos[None, :] > q_pos[:, None] + off)
    if window is not None:
        bad = bad | (k_pos[None, :] < q_pos[:, None] + off - window)
    return np.where(bad, -np.inf, s)


def online_forward(q, k, v, scale, causal, br=64, bc=64, return_state=False, window=None):
    """Returns O [B,Hq,Sq,D], L [B,Hq,Sq] (fp64); with ``return_state`` also (m, l, acc).

    Keys may be longer or shorter than the queries (Skv); the causal diagonal is
    aligned bottom-right, offset = Skv - Sq ("Phase 14", section Causal Mask:
    kv_offset).  ``window`` (>= 0) also hides keys before i + offset - window; KV
    tiles wholly before a Q tile's window are never visited either.  A row that
    sees no key ends with l = 0: its output is 0 and its L is -inf.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off = Skv - Sq
    G = Hq // Hkv
    O = np.zeros((B, Hq, Sq, D))
    L = np.zeros((B, Hq, Sq))
    M = np.zeros((B, Hq, Sq))
    ELL = np.zeros((B, Hq, Sq))
    ACC = np.zeros((B, Hq, Sq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            Kh, Vh = _f64(k[b, g]), _f64(v[b, g])
            for i0 in range(0, Sq, br):
                i1 = min(i0 + br, Sq)
                Qi = _f64(q[b, h, i0:i1])
                q_pos = np.arange(i0, i1)
                m = np.full(i1 - i0, -np.inf)
                ell = np.zeros(i1 - i0)
                acc = np.zeros((i1 - i0, D))
                first = 0 if window is None else max(0, i0 + off - window) // bc * bc
                for j0 in range(first, Skv, bc):
                    if causal and j0 > i1 - 1 + off:
                        break                                   # tile-level causal skip
                    j1 = min(j0 + bc, Skv)
                    s = scale * (Qi @ Kh[j0:j1].T)
                    s = _mask(s, q_pos, np.arange(j0, j1), causal, Skv, off, window)
                    m_new = np.maximum(m, s.max(axis=1))
                    ref = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - ref)
                    p = np.where(np.isfinite(s), np.exp(s - ref[:, None]), 0.0)
                    ell = ell * alpha + p.sum(axis=1)
                    acc = acc * alpha[:, None] + p @ Vh[j0:j1]
                    m = m_new
                seen = ell > 0
                O[b, h, i0:i1] = np.where(seen[:, None], acc / np.where(seen, ell, 1.0)[:, None], 0.0)
                with np.errstate(divide="ignore"):
                    L[b, h, i0:i1] = np.where(seen, m + np.log(np.where(seen, ell, 1.0)), -np.inf)
                M[b, h, i0:i1], ELL[b, h, i0:i1], ACC[b, h, i0:i1] = m, ell, acc
    if return_state:
        return O, L, (M, ELL, ACC)
    return O, L


def online_backward(q, k, v, o, lse, do, scale, causal, br=64, bc=64, window=None):
    """dQ [B,Hq,Sq,D], dK, dV [B,Hkv,Skv,D] (fp64) from the forward's O and L.

    Masks as in ``online_forward``; for a KV tile only the Q tiles that can see
    one of its keys are visited (from the first row at or after j0 - offset, to
    the last row whose window still reaches the tile's last key)."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off = Skv - Sq
    G = Hq // Hkv
    o, lse, do = _f64(o), _f64(lse), _f64(do)
    Dvec = (do * o).sum(axis=-1)                               # first pass: D = rowsum(dO * O)
    dQ = np.zeros((B, Hq, Sq, D))
    dK = np.zeros((B, Hkv, Skv, D))
    dV = np.zeros((B, Hkv, Skv, D))
    for b in range(B):
        for g in range(Hkv):
            Kh, Vh = _f64(k[b, g]), _f64(v[b, g])
            for j0 in range(0, Skv, bc):
                j1 = min(j0 + bc, Skv)
                k_pos = np.arange(j0, j1)
                Kj, Vj = Kh[j0:j1], Vh[j0:j1]
                dKj = np.zeros((j1 - j0, D))
                dVj = np.zeros((j1 - j0, D))
                for h in range(g * G, (g + 1) * G):
                    first = (max(0, j0 - off) // br) * br if causal else 0
                    last = Sq if window is None else min(Sq, j1 - 1 - off + window + 1)
                    for i0 in range(first, last, br):
                        i1 = min(i0 + br, Sq)
                        Qi = _f64(q[b, h, i0:i1])
                        dOi = do[b, h, i0:i1]
                        s = scale * (Qi @ Kj.T)
                        s = _mask(s, np.arange(i0, i1), k_pos, causal, Skv, off, window)
                        with np.errstate(invalid="ignore"):
                            p = np.where(np.isfinite(s), np.exp(s - lse[b, h, i0:i1, None]), 0.0)
                        dVj += p.T @ dOi
                        dp = dOi @ Vj.T
                        ds = p * (dp - Dvec[b, h, i0:i1, None])
                        dQ[b, h, i0:i1] += scale * (ds @ Kj)
                        dKj += scale * (ds.T @ Qi)
                dK[b, g, j0:j1] = dKj
                dV[b, g, j0:j1] = dVj
    return dQ, dK, dV
