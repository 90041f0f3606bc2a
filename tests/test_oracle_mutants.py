"""Planted mistakes in copies of the oracle must be caught by its pins (CPU only).

Each mutant is the oracle's own source with one plausible slip (a dropped term,
a wrong sign, an off-by-one mask, a transposed operand, a wrong head mapping),
executed as a fresh module.  The real oracle is never modified.  The test
passes when at least one pin rejects every mutant.
"""
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(fname, old=None, new=None):
    with open(os.path.join(ROOT, "oracle", fname)) as f:
        src = f.read()
    if old is not None:
        assert src.count(old) >= 1, f"mutation anchor not found in {fname}: {old!r}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant_" + fname[:-3])
    exec(compile(src, fname, "exec"), mod.__dict__)
    return mod


def _pins_hold(dense, tiled):
    """A compact subset of the pins; False as soon as one of them fails."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, S, D = 1, 4, 2, 19, 4
    q = rng.standard_normal((B, Hq, S, D)) * 2
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    do = rng.standard_normal((B, Hq, S, D))
    scale = 0.6
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale, enable_gqa=True)
    out.backward(torch.tensor(do))
    ref = {"o": out.detach().numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}
    try:
        with np.errstate(all="ignore"):
            g = dense.sdpa_backward(q, k, v, do, scale, True)
            Od, Ld = dense.sdpa_forward(q, k, v, scale, True, row_block=7)
            Or, Lr = dense.sdpa_forward_rows(q, k, v, scale, True, 0, 3, np.arange(S))
            dqr = dense.sdpa_dq_rows(q, k, v, do, scale, True, 0, 3, np.arange(S))
            O, L = tiled.online_forward(q, k, v, scale, True, 5, 3)
            dq, dk, dv = tiled.online_backward(q, k, v, O, L, do, scale, True, 5, 3)
    except Exception:
        return False
    ok = all(np.allclose(g[n], ref[n], atol=1e-10) for n in ref)
    ok &= np.allclose(Od, ref["o"], atol=1e-10) and np.allclose(Ld, g["lse"], atol=1e-10)
    ok &= np.allclose(Or, ref["o"][0, 3], atol=1e-10) and np.allclose(Lr, g["lse"][0, 3], atol=1e-10)
    ok &= np.allclose(dqr, ref["dq"][0, 3], atol=1e-10)
    ok &= np.allclose(O, ref["o"], atol=1e-10) and np.allclose(L, g["lse"], atol=1e-10)
    ok &= all(np.allclose(a, ref[n], atol=1e-10) for a, n in zip((dq, dk, dv), ("dq", "dk", "dv")))
    # longer keys (bottom-right causal alignment) with a sliding window, against an explicit mask
    Sq, Skv, win = 13, 19, 4
    q2, k2, v2, do2 = q[:, :, :Sq], rng.standard_normal((B, Hkv, Skv, D)), rng.standard_normal((B, Hkv, Skv, D)), do[:, :, :Sq]
    i, j = np.arange(Sq)[:, None], np.arange(Skv)[None, :]
    mask = torch.tensor((j <= i + Skv - Sq) & (j >= i + Skv - Sq - win))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q2, k2, v2))
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1),
                                         attn_mask=mask, scale=scale)
    out.backward(torch.tensor(do2))
    ref2 = {"o": out.detach().numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}
    try:
        with np.errstate(all="ignore"):
            g2 = dense.sdpa_backward(q2, k2, v2, do2, scale, True, window=win)
            O2, L2 = tiled.online_forward(q2, k2, v2, scale, True, 4, 3, window=win)
            t2 = tiled.online_backward(q2, k2, v2, O2, L2, do2, scale, True, 4, 3, window=win)
    except Exception:
        return False
    ok &= all(np.allclose(g2[n], ref2[n], atol=1e-10) for n in ref2)
    ok &= np.allclose(O2, ref2["o"], atol=1e-10) and np.allclose(L2, g2["lse"], atol=1e-10)
    ok &= all(np.allclose(a, ref2[n], atol=1e-10) for a, n in zip(t2, ("dq", "dk", "dv")))
    # linear position bias on the same longer-key windowed problem, against torch with the
    # bias as an additive float mask
    slopes = [0.5, 0.125, 2.0, 0.25]
    bias = np.stack([np.where((j <= i + Skv - Sq) & (j >= i + Skv - Sq - win), -a * np.abs(i + Skv - Sq - j),
                              -np.inf) for a in slopes])[None]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q2, k2, v2))
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1),
                                         attn_mask=torch.tensor(bias), scale=scale)
    out.backward(torch.tensor(do2))
    ref3 = {"o": out.detach().numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}
    try:
        with np.errstate(all="ignore"):
            g3 = dense.sdpa_backward(q2, k2, v2, do2, scale, True, window=win, alibi=slopes)
            O3, L3 = tiled.online_forward(q2, k2, v2, scale, True, 4, 3, window=win, alibi=slopes)
            t3 = tiled.online_backward(q2, k2, v2, O3, L3, do2, scale, True, 4, 3, window=win, alibi=slopes)
    except Exception:
        return False
    ok &= all(np.allclose(g3[n], ref3[n], atol=1e-10) for n in ref3)
    ok &= np.allclose(O3, ref3["o"], atol=1e-10) and np.allclose(L3, g3["lse"], atol=1e-10)
    ok &= all(np.allclose(a, ref3[n], atol=1e-10) for a, n in zip(t3, ("dq", "dk", "dv")))
    # the bias without the causal mask (keys on both sides of the diagonal)
    bias = np.stack([-a * np.abs(i + Skv - Sq - j) for a in slopes])[None]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q2, k2, v2))
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1),
                                         attn_mask=torch.tensor(bias), scale=scale)
    out.backward(torch.tensor(do2))
    ref4 = {"o": out.detach().numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}
    try:
        with np.errstate(all="ignore"):
            g4 = dense.sdpa_backward(q2, k2, v2, do2, scale, False, alibi=slopes)
            O4, L4 = tiled.online_forward(q2, k2, v2, scale, False, 4, 3, alibi=slopes)
            t4 = tiled.online_backward(q2, k2, v2, O4, L4, do2, scale, False, 4, 3, alibi=slopes)
    except Exception:
        return False
    ok &= all(np.allclose(g4[n], ref4[n], atol=1e-10) for n in ref4)
    ok &= np.allclose(O4, ref4["o"], atol=1e-10) and np.allclose(L4, g4["lse"], atol=1e-10)
    ok &= all(np.allclose(a, ref4[n], atol=1e-10) for a, n in zip(t4, ("dq", "dk", "dv")))
    return bool(ok)


def test_unmutated_oracle_passes():
    assert _pins_hold(_load("dense.py"), _load("tiled.py"))


DENSE_MUTANTS = [
    ("sc = scale * (q_rows @ k_head[:ncols].T)", "sc = (q_rows @ k_head[:ncols].T)"),
    ("vis &= j <= i + offset", "vis &= j < i + offset"),
    ("e = np.exp(sc - m)", "e = np.exp(sc)"),
    ("(m + np.log(np.where(z > 0, z, 1.0)))[:, 0]", "(np.log(np.where(z > 0, z, 1.0)))[:, 0]"),
    ("vis &= j >= i + offset - window", "vis &= j > i + offset - window"),
    ("return h // (Hq // Hkv)", "return h % Hkv"),
    ("dP - (P * dP).sum(axis=1, keepdims=True)", "dP + (P * dP).sum(axis=1, keepdims=True)"),
    ("dP = do_blk @ vh[:nc].T", "dP = do_blk @ vh[:nc].T * 0.5"),
    ('out["dq"][b, h, r0:r1] = scale * (dS @ kh[:nc])', 'out["dq"][b, h, r0:r1] = (dS @ kh[:nc])'),
    ("dk[:nc] += scale * (dS.T @ qh[r0:r1])", "dk[:nc] += scale * (P.T @ qh[r0:r1])"),
    ("dv[:nc] += P.T @ _f64(do[b, h, r0:r1])", "dv[:nc] += dS.T @ _f64(do[b, h, r0:r1])"),
    ("return h // (Hq // Hkv)", "return h % Hkv"),
    ("sc = sc + alibi_bias(rows, np.arange(ncols), slope, offset)", "sc = sc - alibi_bias(rows, np.arange(ncols), slope, offset)"),
    ("return -float(slope) * np.abs(i + offset - j).astype(np.float64)", "return -float(slope) * np.abs(i - j).astype(np.float64)"),
    ("return -float(slope) * np.abs(i + offset - j).astype(np.float64)", "return -float(slope) * (i + offset - j).astype(np.float64)"),
    ("return None if alibi is None else float(alibi[h])", "return None if alibi is None else float(alibi[0])"),
]

TILED_MUTANTS = [
    ("self.l *= alpha", "self.l *= 1.0"),                                   # l not rescaled
    ("self.acc *= alpha[:, None]", "self.acc *= 1.0"),                      # acc not rescaled
    ("hi = min(Skv, i1 + off) if causal else Skv", "hi = min(Skv, i0 + off + 1) if causal else Skv"),
    ("vis &= kk >= qq + off - window", "vis &= kk > qq + off - window"),
    ("stop = Sq if window is None else min(Sq, j1 - 1 - off + window + 1)",
     "stop = Sq if window is None else min(Sq, j1 - 1 - off + window)"),
    ("lse[seen] = self.m[seen] + np.log(self.l[seen])", "lse[seen] = np.log(self.l[seen])"),
    ("vis &= kk <= qq + off", "vis &= kk < qq + off"),
    ("p[vis] = np.exp((s - lse[b, h, i0:i1, None])[vis])", "p[vis] = np.exp(s[vis])"),
    ("ds = p * (dp - rowdot[b, h, i0:i1, None])", "ds = p * (dp + rowdot[b, h, i0:i1, None])"),
    ("dQ[b, h, i0:i1] += scale * (ds @ Kt)", "dQ[b, h, i0:i1] += scale * (p @ Kt)"),
    ("gK += scale * (ds.T @ Qblk)", "gK += (ds.T @ Qblk)"),
    ("first = (max(0, j0 - off) // br) * br if causal else 0", "first = (j0 // br + 1) * br if causal else 0"),
    ('rowdot = np.einsum("bhsd,bhsd->bhs", do, o)', 'rowdot = 0 * np.einsum("bhsd,bhsd->bhs", do, o)'),
    ("kv = h // G\n            Kh, Vh", "kv = h % Hkv\n            Kh, Vh"),
    ("weight[vis] = np.exp((logits - self.m[:, None])[vis])", "weight[vis] = np.exp(logits[vis])"),
    ("gV += p.T @ dOblk", "gV += p.T @ dOblk * 0.5"),
    ("dist = np.abs((q_pos[:, None] + off) - k_pos[None, :])", "dist = np.abs(q_pos[:, None] - k_pos[None, :])"),
    ("logits = logits + _tile_bias(q_pos, k_pos, float(alibi[h]), off)", "logits = logits + _tile_bias(q_pos, k_pos, float(alibi[kv]), off)"),
    ("s = s + _tile_bias(np.arange(i0, i1), k_pos, float(alibi[h]), off)", "s = s + _tile_bias(np.arange(i0, i1), k_pos, float(alibi[h]), -off)"),
]


@pytest.mark.parametrize("old,new", DENSE_MUTANTS)
def test_dense_mutant_is_caught(old, new):
    assert not _pins_hold(_load("dense.py", old, new), _load("tiled.py"))


@pytest.mark.parametrize("old,new", TILED_MUTANTS)
def test_tiled_mutant_is_caught(old, new):
    assert not _pins_hold(_load("dense.py"), _load("tiled.py", old, new))
