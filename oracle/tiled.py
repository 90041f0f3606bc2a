"""Tiled fp64 form: the flash method's own steps, one KV tile at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Forward (``online_forward``).  The loop order is FA2's: query blocks outside,
KV tiles inside ("Phase 14: Flash Attention 2 for SM120 — Design Document",
section "FA2 算法").  A block of query rows carries the online-softmax state of
"Phase T14: 融合 Flash-Attention Kernel — Design Document" (section "什么是
flash-attention"), kept here in a ``RowState``:

* m: the largest visible logit seen so far, per row (the reference point);
* l: the sum of exp(logit - m) over the visible keys seen so far;
* acc: the same weights times the value rows, summed.

A KV tile is folded in two steps.  First the reference moves up to the tile's
maximum, if that is larger, and l and acc are multiplied by exp(m_old - m_new),
so they stay sums relative to the current m.  Then the tile's own weights
exp(logit - m) are added to l, and the weights times the tile's V rows to acc.
At the end O = acc / l and the logsumexp is L = m + log l (decision ②: the state
the backward keeps).

Masking is by a visibility array: an invisible (query, key) pair contributes no
weight, and a row with no visible key so far keeps m = -inf and zero sums.  Its
rescale factor is taken as 1, so exp(-inf - (-inf)) never has to be evaluated.
"FlashAttention 与 SDPA Backend" (section 可运行的 online-softmax reference) states
the same requirement: a fully masked tile must give weight 0, not NaN.

Tile-level causal skip ("Phase 14", section "Causal Mask"; the udemi.tech
"Flash Attention" pseudocode stops its KV loop at the diagonal): a query block
visits only the KV tiles that start before the last key its last row can see.
With a left window it also starts at the first tile its first row can see.
Partial last tiles end at min(start + size, N).

Backward (``online_backward``): the recompute formulas of "Phase T14" (section
"什么是 flash-attention") and decision ③.  The row dot products
D[i] = sum_d dO[i, d] O[i, d] come first.  Then, for every KV tile and every
query block that can see it:

    s  = scale Q_blk K_tile^T,   p = exp(s - L) on visible pairs, 0 elsewhere
    dV_tile += p^T dO_blk,       dp = dO_blk V_tile^T,   ds = p (dp - D)
    dQ_blk  += scale ds K_tile,  dK_tile += scale ds^T Q_blk

GQA: the query heads of a group are visited inside the KV tile's loop, so dK
and dV of the shared KV head sum over the group (chain rule; the pages' GQA
section gives only the forward mapping).

ALiBi (``alibi``: one slope per query head): each tile's scores get
-slope * |i + offset - j| added before the mask, the reading stated in
``dense``; it is written out here again, on the tile's own indices.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _visible(q_pos, k_pos, causal, off, window):
    """Visibility of keys k_pos to queries q_pos: causal j <= i + off (bottom-right
    alignment, off = Skv - Sq), window j >= i + off - window."""
    qq = q_pos[:, None]
    kk = k_pos[None, :]
    vis = np.ones((q_pos.size, k_pos.size), dtype=bool)
    if causal:
        vis &= kk <= qq + off
    if window is not None:
        vis &= kk >= qq + off - window
    return vis


class RowState:
    """Online-softmax state (m, l, acc) of a block of n query rows, head dim D."""

    def __init__(self, n, D):
        self.m = np.full(n, -np.inf)
        self.l = np.zeros(n)
        self.acc = np.zeros((n, D))

    def rescale_to(self, m_new):
        """Make m_new (>= m, row by row) the reference: the old sums shrink by
        exp(m - m_new).  Rows still at -inf have empty sums and keep factor 1."""
        alpha = np.ones_like(self.m)
        live = np.isfinite(m_new)
        alpha[live] = np.exp(self.m[live] - m_new[live])
        self.l *= alpha
        self.acc *= alpha[:, None]
        self.m = m_new

    def absorb(self, logits, vis, v_tile):
        """Fold one KV tile into the state: logits and vis are (n, keys), v_tile (keys, D)."""
        tile_top = np.where(vis, logits, -np.inf).max(axis=1)
        self.rescale_to(np.maximum(self.m, tile_top))
        weight = np.zeros_like(logits)
        weight[vis] = np.exp((logits - self.m[:, None])[vis])
        self.l += weight.sum(axis=1)
        self.acc += weight @ v_tile

    def result(self):
        """(O, L) of the rows.  A row that saw no key has an empty softmax: O = 0, L = -inf."""
        seen = self.l > 0
        out = np.zeros_like(self.acc)
        out[seen] = self.acc[seen] / self.l[seen][:, None]
        lse = np.full(self.m.shape, -np.inf)
        lse[seen] = self.m[seen] + np.log(self.l[seen])
        return out, lse


def _tile_bias(q_pos, k_pos, slope, off):
    """-slope * distance from each query's diagonal position to each key of the tile."""
    dist = np.abs((q_pos[:, None] + off) - k_pos[None, :])
    return -slope * dist


def online_forward(q, k, v, scale, causal, br=64, bc=64, return_state=False, window=None, alibi=None):
    """Returns O [B,Hq,Sq,D], L [B,Hq,Sq] (fp64); with ``return_state`` also the final
    (m, l, acc) of every row.

    Keys may be longer or shorter than the queries (Skv); the causal diagonal is
    aligned bottom-right, offset = Skv - Sq ("Phase 14", section Causal Mask:
    kv_offset).  ``window`` (>= 0) also hides keys before i + offset - window.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off = Skv - Sq
    G = Hq // Hkv
    O = np.zeros((B, Hq, Sq, D))
    L = np.zeros((B, Hq, Sq))
    state = (np.zeros((B, Hq, Sq)), np.zeros((B, Hq, Sq)), np.zeros((B, Hq, Sq, D)))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            Kh, Vh = _f64(k[b, kv]), _f64(v[b, kv])
            for i0 in range(0, Sq, br):
                i1 = min(i0 + br, Sq)
                rows = RowState(i1 - i0, D)
                Qblk = _f64(q[b, h, i0:i1])
                q_pos = np.arange(i0, i1)
                # KV tiles that some row of the block can see: [lo, hi)
                hi = min(Skv, i1 + off) if causal else Skv
                lo = 0 if window is None else max(0, i0 + off - window) // bc * bc
                for j0 in range(lo, hi, bc):
                    j1 = min(j0 + bc, Skv)
                    k_pos = np.arange(j0, j1)
                    vis = _visible(q_pos, k_pos, causal, off, window)
                    logits = scale * (Qblk @ Kh[j0:j1].T)
                    if alibi is not None:
                        logits = logits + _tile_bias(q_pos, k_pos, float(alibi[h]), off)
                    rows.absorb(logits, vis, Vh[j0:j1])
                O[b, h, i0:i1], L[b, h, i0:i1] = rows.result()
                for dst, val in zip(state, (rows.m, rows.l, rows.acc)):
                    dst[b, h, i0:i1] = val
    if return_state:
        return O, L, state
    return O, L


def online_backward(q, k, v, o, lse, do, scale, causal, br=64, bc=64, window=None, alibi=None):
    """dQ [B,Hq,Sq,D], dK, dV [B,Hkv,Skv,D] (fp64) from the forward's O and L.

    Masks as in ``online_forward``.  For a KV tile only the query blocks that can
    see one of its keys are visited: from the block holding row j0 - offset (causal)
    to the last row whose window still reaches the tile's last key."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off = Skv - Sq
    G = Hq // Hkv
    o, lse, do = _f64(o), _f64(lse), _f64(do)
    rowdot = np.einsum("bhsd,bhsd->bhs", do, o)              # D[i] = sum_d dO[i, d] O[i, d]
    dQ = np.zeros((B, Hq, Sq, D))
    dK = np.zeros((B, Hkv, Skv, D))
    dV = np.zeros((B, Hkv, Skv, D))
    for b in range(B):
        for kv in range(Hkv):
            Kh, Vh = _f64(k[b, kv]), _f64(v[b, kv])
            for j0 in range(0, Skv, bc):
                j1 = min(j0 + bc, Skv)
                Kt, Vt = Kh[j0:j1], Vh[j0:j1]
                k_pos = np.arange(j0, j1)
                gK = np.zeros((j1 - j0, D))
                gV = np.zeros((j1 - j0, D))
                first = (max(0, j0 - off) // br) * br if causal else 0
                stop = Sq if window is None else min(Sq, j1 - 1 - off + window + 1)
                for h in range(kv * G, (kv + 1) * G):
                    for i0 in range(first, stop, br):
                        i1 = min(i0 + br, Sq)
                        Qblk = _f64(q[b, h, i0:i1])
                        dOblk = do[b, h, i0:i1]
                        vis = _visible(np.arange(i0, i1), k_pos, causal, off, window)
                        s = scale * (Qblk @ Kt.T)
                        if alibi is not None:
                            s = s + _tile_bias(np.arange(i0, i1), k_pos, float(alibi[h]), off)
                        p = np.zeros_like(s)
                        p[vis] = np.exp((s - lse[b, h, i0:i1, None])[vis])
                        gV += p.T @ dOblk
                        dp = dOblk @ Vt.T
                        ds = p * (dp - rowdot[b, h, i0:i1, None])
                        dQ[b, h, i0:i1] += scale * (ds @ Kt)
                        gK += scale * (ds.T @ Qblk)
                dK[b, kv, j0:j1] = gK
                dV[b, kv, j0:j1] = gV
    return dQ, dK, dV
