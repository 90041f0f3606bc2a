"""Pins for the fp64 CPU oracle (CPU only).

Each check ties the oracle to something other than itself: a hand-derived
worked example, closed forms, invariants of softmax attention, finite
differences, brute force on tiny inputs, or PyTorch's own fp64 CPU attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def rand_qkvdo(B, Hq, Hkv, S, D, seed, std=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, S, D)) * std
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    do = r.standard_normal((B, Hq, S, D))
    return q, k, v, do


# ---------------------------------------------------------------- worked example

def _golden():
    with open(os.path.join(HERE, "golden", "worked_example_s3_d2.json")) as f:
        doc = json.load(f)
    env = {"__builtins__": {}, "ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4),
           "ln5": math.log(5), "ln8": math.log(8)}

    def ev(x):
        return [ev(y) for y in x] if isinstance(x, list) else eval(x, env)  # expressions written in the fixture

    inp = {k: np.array(ev(v))[None, None] for k, v in doc["inputs_expr"].items()}
    exp = {c: {k: np.array(ev(v))[None, None] for k, v in doc[c + "_expr"].items()}
           for c in ("causal", "noncausal")}
    # the stored floats are the same expressions evaluated once
    for c in exp:
        for k in exp[c]:
            np.testing.assert_allclose(exp[c][k][0, 0], np.array(doc[c][k]), atol=1e-15)
    return doc["scale"], inp, exp


@pytest.mark.parametrize("causal", [True, False])
def test_worked_example_dense(causal):
    scale, inp, exp = _golden()
    e = exp["causal" if causal else "noncausal"]
    O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], scale, causal)
    np.testing.assert_allclose(O, e["o"], atol=1e-14)
    np.testing.assert_allclose(L, e["lse"], atol=1e-14)
    g = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(g[key], e[key], atol=1e-14, err_msg=key)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("br,bc", [(1, 1), (2, 1), (1, 2), (2, 2), (3, 3)])
def test_worked_example_tiled(causal, br, bc):
    scale, inp, exp = _golden()
    e = exp["causal" if causal else "noncausal"]
    O, L = oracle.online_forward(inp["q"], inp["k"], inp["v"], scale, causal, br, bc)
    np.testing.assert_allclose(O, e["o"], atol=1e-14)
    np.testing.assert_allclose(L, e["lse"], atol=1e-14)
    dq, dk, dv = oracle.online_backward(inp["q"], inp["k"], inp["v"], O, L, inp["do"], scale, causal, br, bc)
    np.testing.assert_allclose(dq, e["dq"], atol=1e-14)
    np.testing.assert_allclose(dk, e["dk"], atol=1e-14)
    np.testing.assert_allclose(dv, e["dv"], atol=1e-14)


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, do, scale, causal):
    """Scalar loops over every (b, h, i, j): independent of both oracle forms."""
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(S):
                js = [j for j in range(S) if not (causal and j > i)]
                s = {j: scale * sum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) for j in js}
                z = sum(math.exp(s[j]) for j in js)
                p = {j: math.exp(s[j]) / z for j in js}
                L[b, h, i] = math.log(z)
                for d in range(D):
                    O[b, h, i, d] = sum(p[j] * v[b, g, j, d] for j in js)
                dp = {j: sum(do[b, h, i, d] * v[b, g, j, d] for d in range(D)) for j in js}
                pdp = sum(p[j] * dp[j] for j in js)
                for j in js:
                    ds = p[j] * (dp[j] - pdp)
                    for d in range(D):
                        dq[b, h, i, d] += scale * ds * k[b, g, j, d]
                        dk[b, g, j, d] += scale * ds * q[b, h, i, d]
                        dv[b, g, j, d] += p[j] * do[b, h, i, d]
    return O, L, dq, dk, dv


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    q, k, v, do = rand_qkvdo(1, 4, 2, 6, 3, seed=11)
    scale = 0.7
    O, L, dq, dk, dv = _brute(q, k, v, do, scale, causal)
    g = oracle.sdpa_backward(q, k, v, do, scale, causal)
    for name, ref in (("o", O), ("lse", L), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(g[name], ref, atol=1e-13, err_msg=name)
    Ot, Lt = oracle.online_forward(q, k, v, scale, causal, 4, 4)
    np.testing.assert_allclose(Ot, O, atol=1e-13)
    np.testing.assert_allclose(Lt, L, atol=1e-13)
    t = oracle.online_backward(q, k, v, Ot, Lt, do, scale, causal, 4, 4)
    for got, ref in zip(t, (dq, dk, dv)):
        np.testing.assert_allclose(got, ref, atol=1e-13)


# ---------------------------------------------------------------- library routine

def _torch_reference(q, k, v, do, scale, causal):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=G > 1)
    out.backward(torch.tensor(do, dtype=torch.float64))
    kr = tk.detach().repeat_interleave(G, dim=1)
    vr = tv.detach().repeat_interleave(G, dim=1)
    o2, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq.detach(), kr, vr, 0.0, causal, scale=scale)[:2]
    np.testing.assert_allclose(o2.numpy(), out.detach().numpy(), atol=1e-12)
    return out.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 2, 2, 37, 8), (2, 4, 1, 20, 16), (1, 6, 3, 65, 4)])
def test_against_torch_fp64(B, Hq, Hkv, S, D, causal):
    q, k, v, do = rand_qkvdo(B, Hq, Hkv, S, D, seed=S + D)
    scale = 1.0 / math.sqrt(D)
    O, L, dq, dk, dv = _torch_reference(q, k, v, do, scale, causal)
    g = oracle.sdpa_backward(q, k, v, do, scale, causal)
    for name, ref in (("o", O), ("lse", L), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(g[name], ref, atol=1e-11, rtol=1e-11, err_msg=name)
    Ot, Lt = oracle.online_forward(q, k, v, scale, causal, 16, 8)
    np.testing.assert_allclose(Ot, O, atol=1e-11)
    np.testing.assert_allclose(Lt, L, atol=1e-11)
    for got, ref in zip(oracle.online_backward(q, k, v, Ot, Lt, do, scale, causal, 16, 8), (dq, dk, dv)):
        np.testing.assert_allclose(got, ref, atol=1e-11, rtol=1e-11)


# ---------------------------------------------------------------- tiled == dense

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [1, 5, 17, 70])
@pytest.mark.parametrize("br,bc", [(1, 1), (3, 3), (16, 16), (64, 64), (16, 3), (3, 16), (70, 70)])
def test_tiled_equals_dense(S, br, bc, causal):
    q, k, v, do = rand_qkvdo(1, 4, 2, S, 8, seed=S * 7 + br + bc, std=2.0)
    scale = 0.35
    g = oracle.sdpa_backward(q, k, v, do, scale, causal)
    O, L = oracle.online_forward(q, k, v, scale, causal, br, bc)
    np.testing.assert_allclose(O, g["o"], atol=1e-12)
    np.testing.assert_allclose(L, g["lse"], atol=1e-12)
    dq, dk, dv = oracle.online_backward(q, k, v, O, L, do, scale, causal, br, bc)
    np.testing.assert_allclose(dq, g["dq"], atol=1e-12)
    np.testing.assert_allclose(dk, g["dk"], atol=1e-12)
    np.testing.assert_allclose(dv, g["dv"], atol=1e-12)


def test_online_state_shapes():
    q, k, v, _ = rand_qkvdo(1, 2, 2, 7, 4, seed=71)
    O, L, (m, ell, acc) = oracle.online_forward(q, k, v, 0.5, True, 7, 3, return_state=True)
    assert m.shape == ell.shape == (1, 2, 7) and acc.shape == q.shape
    np.testing.assert_allclose(acc / ell[..., None], O, atol=1e-15)
    np.testing.assert_allclose(m + np.log(ell), L, atol=1e-15)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
def test_row0_exact(causal):
    q, k, v, do = rand_qkvdo(2, 4, 2, 33, 8, seed=5)
    scale = 0.125
    O, L = oracle.sdpa_forward(q, k, v, scale, causal=True)
    G = 2
    for b in range(2):
        for h in range(4):
            assert np.array_equal(O[b, h, 0], v[b, h // G, 0])          # p = 1 exactly
            np.testing.assert_allclose(L[b, h, 0], scale * q[b, h, 0] @ k[b, h // G, 0], atol=1e-15)
    Ot, _ = oracle.online_forward(q, k, v, scale, True, 8, 8)
    assert np.array_equal(Ot[:, :, 0], np.repeat(v[:, :, 0], G, axis=1))


def test_zero_query_uniform_weights():
    B, Hq, Hkv, S, D = 1, 4, 2, 23, 5
    _, k, v, do = rand_qkvdo(B, Hq, Hkv, S, D, seed=8)
    q = np.zeros((B, Hq, S, D))
    G = Hq // Hkv
    i = np.arange(S)
    for form in ("dense", "tiled"):
        if form == "dense":
            g = oracle.sdpa_backward(q, k, v, do, 0.3, True)
            O, L, dq, dk, dv = g["o"], g["lse"], g["dq"], g["dk"], g["dv"]
        else:
            O, L = oracle.online_forward(q, k, v, 0.3, True, 5, 4)
            dq, dk, dv = oracle.online_backward(q, k, v, O, L, do, 0.3, True, 5, 4)
        mean_v = np.cumsum(v, axis=2) / (i + 1)[None, None, :, None]
        np.testing.assert_allclose(O, np.repeat(mean_v, G, axis=1), atol=1e-13)
        np.testing.assert_allclose(L, np.broadcast_to(np.log(i + 1.0), L.shape), atol=1e-13)
        assert np.all(dk == 0.0)                                            # Q = 0 gives dK = 0 exactly
        # dV[j] = sum over the group's heads and rows i >= j of dO[i] / (i + 1)
        w = do / (i + 1)[None, None, :, None]
        suffix = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
        np.testing.assert_allclose(dv, suffix.reshape(B, Hkv, G, S, D).sum(axis=2), atol=1e-12)


def test_zero_key_gives_zero_dq():
    q, _, v, do = rand_qkvdo(1, 2, 1, 19, 4, seed=9)
    k = np.zeros((1, 1, 19, 4))
    g = oracle.sdpa_backward(q, k, v, do, 0.5, True)
    assert np.all(g["dq"] == 0.0)
    O, L = oracle.online_forward(q, k, v, 0.5, True, 4, 4)
    assert np.all(oracle.online_backward(q, k, v, O, L, do, 0.5, True, 4, 4)[0] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_constant_values(causal):
    q, k, _, do = rand_qkvdo(1, 2, 2, 29, 6, seed=10)
    c = np.random.default_rng(1).standard_normal(6)
    v = np.broadcast_to(c, (1, 2, 29, 6)).copy()
    g = oracle.sdpa_backward(q, k, v, do, 0.4, causal)
    np.testing.assert_allclose(g["o"], np.broadcast_to(c, g["o"].shape), atol=1e-13)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)
    O, L = oracle.online_forward(q, k, v, 0.4, causal, 8, 8)
    dq, dk, _ = oracle.online_backward(q, k, v, O, L, do, 0.4, causal, 8, 8)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def test_single_position():
    q, k, v, do = rand_qkvdo(2, 4, 2, 1, 8, seed=12)
    scale = 0.25
    g = oracle.sdpa_backward(q, k, v, do, scale, True)
    kr = np.repeat(k, 2, axis=1)
    np.testing.assert_allclose(g["o"], np.repeat(v, 2, axis=1), atol=0)
    np.testing.assert_allclose(g["lse"], scale * (q * kr).sum(-1), atol=1e-15)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_allclose(g["dv"], do.reshape(2, 2, 2, 1, 8).sum(axis=2), atol=1e-15)


@pytest.mark.parametrize("u_scale", [1.0, 40.0])
def test_key_shift(u_scale):
    """Adding u to every key shifts each row's scores by a constant: P, O, dQ unchanged, L += scale q.u."""
    q, k, v, do = rand_qkvdo(1, 2, 2, 31, 8, seed=13)
    u = np.random.default_rng(2).standard_normal(8) * u_scale
    scale = 0.3
    a = oracle.sdpa_backward(q, k, v, do, scale, True)
    b = oracle.sdpa_backward(q, k + u, v, do, scale, True)
    np.testing.assert_allclose(b["o"], a["o"], atol=1e-11)
    np.testing.assert_allclose(b["dq"], a["dq"], atol=1e-10)
    np.testing.assert_allclose(b["lse"], a["lse"] + scale * (q @ u), atol=1e-10)
    Ot, Lt = oracle.online_forward(q, k + u, v, scale, True, 8, 4)
    np.testing.assert_allclose(Ot, a["o"], atol=1e-11)
    np.testing.assert_allclose(Lt, a["lse"] + scale * (q @ u), atol=1e-10)


# ---------------------------------------------------------------- invariants

def test_probability_rows_and_d_identity():
    q, k, v, do = rand_qkvdo(1, 1, 1, 40, 8, seed=14)
    rows = np.arange(40)
    P, L, nc = oracle.softmax_probs(q[0, 0], rows, k[0, 0], 0.35, True)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.triu(P, 1) == 0.0)
    O, _ = oracle.sdpa_forward(q, k, v, 0.35, True)
    dP = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((P * dP).sum(axis=1), (do[0, 0] * O[0, 0]).sum(axis=1), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_gradient_sums(causal):
    q, k, v, do = rand_qkvdo(2, 6, 2, 27, 5, seed=15)
    g = oracle.sdpa_backward(q, k, v, do, 0.45, causal)
    np.testing.assert_allclose(g["dk"].sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dv"].sum(axis=2), do.reshape(2, 2, 3, 27, 5).sum(axis=(2, 3)), atol=1e-12)


def test_gqa_equals_repeated_mha():
    q, k, v, do = rand_qkvdo(1, 8, 2, 21, 4, seed=16)
    G = 4
    a = oracle.sdpa_backward(q, k, v, do, 0.5, True)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    b = oracle.sdpa_backward(q, kr, vr, do, 0.5, True)
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-14)
    np.testing.assert_allclose(a["dq"], b["dq"], atol=1e-14)
    np.testing.assert_allclose(a["dk"], b["dk"].reshape(1, 2, G, 21, 4).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(a["dv"], b["dv"].reshape(1, 2, G, 21, 4).sum(axis=2), atol=1e-13)


def test_last_causal_row_sees_everything():
    q, k, v, _ = rand_qkvdo(1, 2, 2, 18, 4, seed=17)
    Oc, Lc = oracle.sdpa_forward(q, k, v, 0.5, True)
    On, Ln = oracle.sdpa_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(Oc[:, :, -1], On[:, :, -1], atol=1e-15)
    np.testing.assert_allclose(Lc[:, :, -1], Ln[:, :, -1], atol=1e-15)
    assert not np.allclose(Oc[:, :, 0], On[:, :, 0])


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 1, 1, 1, 4), (1, 2, 1, 5, 4), (1, 2, 2, 17, 8)])
def test_finite_differences(B, Hq, Hkv, S, D, causal):
    """Central differences of f = sum(dO * O) in fp64 (the objective of the T14 grad-check)."""
    q, k, v, do = rand_qkvdo(B, Hq, Hkv, S, D, seed=18 + S)
    scale = 1.0 / math.sqrt(D)

    def f(q_, k_, v_):
        return float((oracle.sdpa_forward(q_, k_, v_, scale, causal)[0] * do).sum())

    g = oracle.sdpa_backward(q, k, v, do, scale, causal)
    O, L = oracle.online_forward(q, k, v, scale, causal, 4, 3)
    tiled = dict(zip(("dq", "dk", "dv"), oracle.online_backward(q, k, v, O, L, do, scale, causal, 4, 3)))
    h = 1e-6
    rng = np.random.default_rng(S)
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        idx = [tuple(rng.integers(0, n) for n in arr.shape) for _ in range(12)]
        for ix in idx:
            plus, minus = arr.copy(), arr.copy()
            plus[ix] += h
            minus[ix] -= h
            args_p = {"dq": (plus, k, v), "dk": (q, plus, v), "dv": (q, k, plus)}[name]
            args_m = {"dq": (minus, k, v), "dk": (q, minus, v), "dv": (q, k, minus)}[name]
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(g[name][ix] - fd) <= 1e-7 * max(1.0, abs(fd)), (name, ix, g[name][ix], fd)
            assert abs(tiled[name][ix] - fd) <= 1e-7 * max(1.0, abs(fd)), (name, ix)


# ---------------------------------------------------------------- subset helpers

def test_row_and_group_subsets_match_full():
    q, k, v, do = rand_qkvdo(2, 4, 2, 50, 8, seed=19, std=3.0)
    scale = 0.3
    full = oracle.sdpa_backward(q, k, v, do, scale, True)
    rows = np.array([0, 1, 17, 48, 49])
    Or, Lr = oracle.sdpa_forward_rows(q, k, v, scale, True, 1, 3, rows)
    np.testing.assert_allclose(Or, full["o"][1, 3, rows], atol=1e-13)
    np.testing.assert_allclose(Lr, full["lse"][1, 3, rows], atol=1e-13)
    np.testing.assert_allclose(oracle.sdpa_dq_rows(q, k, v, do, scale, True, 1, 3, rows),
                               full["dq"][1, 3, rows], atol=1e-13)
    sub = oracle.sdpa_backward(q, k, v, do, scale, True, groups=[(1, 0)], row_block=7)
    for key in ("dk", "dv"):
        np.testing.assert_allclose(sub[key][1, 0], full[key][1, 0], atol=1e-12)
        assert np.isnan(sub[key][0, 0]).all()
    np.testing.assert_allclose(sub["dq"][1, :2], full["dq"][1, :2], atol=1e-12)
    O, L = oracle.sdpa_forward(q, k, v, scale, True, heads=[(0, 2)], row_block=9)
    np.testing.assert_allclose(O[0, 2], full["o"][0, 2], atol=1e-13)


def test_workload_inputs_are_on_the_dtype_grid():
    x = make_inputs(1, 2, 1, 8, 4, "bf16", seed=0)
    for a in x.values():
        assert np.all((a.view(np.uint32) & 0xFFFF) == 0)
    y = make_inputs(1, 2, 1, 8, 4, "f16", seed=0)
    for a in y.values():
        assert np.array_equal(a.astype(np.float16).astype(np.float32), a)
    z = make_inputs(1, 2, 1, 8, 4, "bf16", seed=0)
    assert all(np.array_equal(x[key], z[key]) for key in x)


# ---------------------------------------------------------------- cross-length causal, windows, varlen

def _torch_masked(q, k, v, do, scale, causal, window):
    """PyTorch fp64 attention with the same visibility mask written as a boolean matrix."""
    Sq, Skv = q.shape[2], k.shape[2]
    G = q.shape[1] // k.shape[1]
    i, j = np.arange(Sq)[:, None], np.arange(Skv)[None, :]
    vis = np.ones((Sq, Skv), bool)
    if causal:
        vis &= j <= i + Skv - Sq
    if window is not None:
        vis &= j >= i + Skv - Sq - window
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1),
                                         attn_mask=torch.tensor(vis), scale=scale)
    seen = vis.any(axis=1)
    out.backward(torch.tensor(np.where(seen[None, None, :, None], do, 0.0)))
    return vis, out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


MASK_CASES = [  # Sq, Skv, causal, window
    (9, 21, True, None), (21, 9, True, None), (17, 17, True, 5), (12, 30, True, 0),
    (30, 12, False, 4), (16, 16, False, None), (7, 40, True, 11), (25, 25, True, 30),
]


@pytest.mark.parametrize("Sq,Skv,causal,window", MASK_CASES)
def test_masks_against_torch_fp64(Sq, Skv, causal, window):
    r = np.random.default_rng(Sq * 100 + Skv)
    q = r.standard_normal((2, 4, Sq, 8)) * 1.5
    k, v = r.standard_normal((2, 2, Skv, 8)), r.standard_normal((2, 2, Skv, 8))
    do = r.standard_normal((2, 4, Sq, 8))
    scale = 0.4
    vis, O, dq, dk, dv = _torch_masked(q, k, v, do, scale, causal, window)
    seen = vis.any(axis=1)
    g = oracle.sdpa_backward(q, k, v, np.where(seen[None, None, :, None], do, 0.0), scale, causal, window=window)
    np.testing.assert_allclose(g["o"][:, :, seen], O[:, :, seen], atol=1e-12)
    np.testing.assert_allclose(g["dq"], dq, atol=1e-12)
    np.testing.assert_allclose(g["dk"], dk, atol=1e-12)
    np.testing.assert_allclose(g["dv"], dv, atol=1e-12)
    # rows that see no key: empty softmax, O = 0, L = -inf, no gradient
    assert np.all(g["o"][:, :, ~seen] == 0) and np.all(np.isneginf(g["lse"][:, :, ~seen]))
    g2 = oracle.sdpa_backward(q, k, v, do, scale, causal, window=window)
    assert np.all(g2["dq"][:, :, ~seen] == 0)


@pytest.mark.parametrize("Sq,Skv,causal,window", MASK_CASES)
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 3), (16, 8), (64, 64)])
def test_masks_tiled_equals_dense(Sq, Skv, causal, window, br, bc):
    q, k, v, do = rand_qkvdo(1, 2, 1, max(Sq, Skv), 4, seed=Sq + Skv + br, std=2.0)
    q, do = q[:, :, :Sq], do[:, :, :Sq]
    k, v = k[:, :, :Skv], v[:, :, :Skv]
    g = oracle.sdpa_backward(q, k, v, do, 0.5, causal, window=window)
    O, L = oracle.online_forward(q, k, v, 0.5, causal, br, bc, window=window)
    np.testing.assert_allclose(O, g["o"], atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(L), np.isneginf(g["lse"]))
    fin = np.isfinite(g["lse"])
    np.testing.assert_allclose(L[fin], g["lse"][fin], atol=1e-12)
    dq, dk, dv = oracle.online_backward(q, k, v, O, L, do, 0.5, causal, br, bc, window=window)
    np.testing.assert_allclose(dq, g["dq"], atol=1e-12)
    np.testing.assert_allclose(dk, g["dk"], atol=1e-12)
    np.testing.assert_allclose(dv, g["dv"], atol=1e-12)


def test_masks_brute_force():
    r = np.random.default_rng(5)
    Sq, Skv, D, scale, win = 5, 8, 3, 0.7, 2
    q, k, v, do = (r.standard_normal(s) for s in ((1, 1, Sq, D), (1, 1, Skv, D), (1, 1, Skv, D), (1, 1, Sq, D)))
    off = Skv - Sq
    g = oracle.sdpa_backward(q, k, v, do, scale, True, window=win)
    for i in range(Sq):
        js = [j for j in range(Skv) if i + off - win <= j <= i + off]
        s = {j: scale * sum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) for j in js}
        z = sum(math.exp(x) for x in s.values())
        for d in range(D):
            o = sum(math.exp(s[j]) / z * v[0, 0, j, d] for j in js)
            assert abs(g["o"][0, 0, i, d] - o) < 1e-13
        assert abs(g["lse"][0, 0, i] - math.log(z)) < 1e-13


def test_window_zero_sees_one_key():
    """window = 0 under the causal mask: query i sees exactly key i + offset."""
    q, k, v, do = rand_qkvdo(1, 2, 2, 30, 8, seed=41)
    q, do = q[:, :, :12], do[:, :, :12]
    off = 30 - 12
    g = oracle.sdpa_backward(q, k, v, do, 0.3, True, window=0)
    np.testing.assert_array_equal(g["o"], v[:, :, off:])
    np.testing.assert_allclose(g["lse"], 0.3 * (q * k[:, :, off:]).sum(-1), atol=1e-14)
    assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
    np.testing.assert_array_equal(g["dv"][:, :, off:], do)
    assert np.all(g["dv"][:, :, :off] == 0)


def test_single_query_is_full_attention():
    """One query row with the bottom-right causal mask sees every key (a decode step)."""
    q, k, v, do = rand_qkvdo(2, 4, 2, 50, 8, seed=42)
    q1, do1 = q[:, :, -1:], do[:, :, -1:]
    a = oracle.sdpa_backward(q1, k, v, do1, 0.35, True)
    b = oracle.sdpa_backward(q1, k, v, do1, 0.35, False)
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[key], b[key], atol=1e-14)


def test_varlen_equal_lengths_match_dense_batch():
    r = np.random.default_rng(43)
    B, Hq, Hkv, Sq, Skv, D = 3, 4, 2, 11, 17, 8
    q, do = r.standard_normal((B, Hq, Sq, D)), r.standard_normal((B, Hq, Sq, D))
    k, v = r.standard_normal((B, Hkv, Skv, D)), r.standard_normal((B, Hkv, Skv, D))
    dense = oracle.sdpa_backward(q, k, v, do, 0.4, True, window=6)
    pack = lambda x: np.concatenate([x[b] for b in range(B)], axis=1)      # [H, B*S, D]
    cu_q, cu_k = np.arange(B + 1) * Sq, np.arange(B + 1) * Skv
    vl = oracle.sdpa_backward_varlen(pack(q), pack(k), pack(v), pack(do), cu_q, cu_k, 0.4, True, window=6)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(vl[key], pack(dense[key]), atol=1e-13)
    np.testing.assert_allclose(vl["lse"], np.concatenate([dense["lse"][b] for b in range(B)], axis=1), atol=1e-13)
    O, L = oracle.sdpa_forward_varlen(pack(q), pack(k), pack(v), cu_q, cu_k, 0.4, True, window=6)
    np.testing.assert_allclose(O, vl["o"], atol=1e-14)


def test_varlen_ragged_brute_force():
    r = np.random.default_rng(44)
    lq, lk = [3, 0, 5, 1], [4, 2, 5, 6]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = r.standard_normal((2, cu_q[-1], 2)), r.standard_normal((1, cu_k[-1], 2)), r.standard_normal((1, cu_k[-1], 2))
    O, L = oracle.sdpa_forward_varlen(q, k, v, cu_q, cu_k, 0.9, True)
    for b in range(4):
        off = lk[b] - lq[b]
        for h in range(2):
            for i in range(lq[b]):
                js = [j for j in range(lk[b]) if j <= i + off]
                s = [0.9 * float(q[h, cu_q[b] + i] @ k[0, cu_k[b] + j]) for j in js]
                w = np.exp(np.array(s) - max(s))
                ref = (w[:, None] * v[0, [cu_k[b] + j for j in js]]).sum(0) / w.sum()
                np.testing.assert_allclose(O[h, cu_q[b] + i], ref, atol=1e-13)


@pytest.mark.parametrize("Sq,Skv,window", [(4, 7, 2), (6, 3, None), (5, 5, 1)])
def test_masks_finite_differences(Sq, Skv, window):
    r = np.random.default_rng(Sq * 10 + Skv)
    q, k, v = r.standard_normal((1, 2, Sq, 4)), r.standard_normal((1, 1, Skv, 4)), r.standard_normal((1, 1, Skv, 4))
    do = r.standard_normal((1, 2, Sq, 4))

    def f(q_, k_, v_):
        return float((oracle.sdpa_forward(q_, k_, v_, 0.5, True, window=window)[0] * do).sum())

    g = oracle.sdpa_backward(q, k, v, do, 0.5, True, window=window)
    h = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        for ix in np.ndindex(arr.shape):
            if r.random() > 0.3:
                continue
            p, m = arr.copy(), arr.copy()
            p[ix] += h
            m[ix] -= h
            a = {"dq": (p, k, v), "dk": (q, p, v), "dv": (q, k, p)}[name]
            b = {"dq": (m, k, v), "dk": (q, m, v), "dv": (q, k, m)}[name]
            fd = (f(*a) - f(*b)) / (2 * h)
            assert abs(g[name][ix] - fd) <= 1e-7 * max(1.0, abs(fd)), (name, ix)


# ---------------------------------------------------------------- ALiBi (linear position bias)
#
# Reading (the SDPA page only lists ALiBi in its support matrix): query i and key j
# get -a_h * |i + offset - j| added to their scaled score, a_h one slope per query head.

SLOPES4 = [0.5, 0.125, 2.0, 0.0]


def test_alibi_zero_slope_is_no_bias():
    q, k, v, do = rand_qkvdo(1, 4, 2, 23, 8, seed=40)
    for causal in (True, False):
        a = oracle.sdpa_backward(q, k, v, do, 0.4, causal, alibi=[0.0] * 4)
        b = oracle.sdpa_backward(q, k, v, do, 0.4, causal)
        for n in a:
            np.testing.assert_array_equal(a[n], b[n])
        Oa, La = oracle.online_forward(q, k, v, 0.4, causal, 4, 3, alibi=[0.0] * 4)
        Ob, Lb = oracle.online_forward(q, k, v, 0.4, causal, 4, 3)
        np.testing.assert_array_equal(Oa, Ob)
        np.testing.assert_array_equal(La, Lb)


@pytest.mark.parametrize("Sq,Skv,causal", [(40, 40, True), (17, 40, True), (40, 40, False), (25, 31, False)])
def test_alibi_zero_keys_geometric_weights(Sq, Skv, causal):
    """K = 0 leaves the bias alone in the scores: with r = exp(-a), query i weighs key j
    by r^|i + offset - j|.  Causal, the visible keys are j <= i + offset, so the weights are
    1, r, r^2, ... back from the diagonal and L_i = log((1 - r^(n)) / (1 - r)) with n the
    number of visible keys; non-causal, the two sides of the diagonal add up the same way."""
    D = 4
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, 4, Sq, D))
    k = np.zeros((1, 4, Skv, D))
    v = rng.standard_normal((1, 4, Skv, D))
    off = Skv - Sq
    O, L = oracle.sdpa_forward(q, k, v, 0.5, causal, alibi=SLOPES4[:3] + [0.3])
    Ot, Lt = oracle.online_forward(q, k, v, 0.5, causal, 5, 4, alibi=SLOPES4[:3] + [0.3])
    for h, a in enumerate(SLOPES4[:3] + [0.3]):
        r = math.exp(-a)

        def geo(n):  # 1 + r + ... + r^(n-1)
            return (1 - r ** n) / (1 - r)

        for i in range(Sq):
            d = i + off  # the diagonal key of row i
            left = min(d, Skv - 1)
            if causal:
                z = geo(d + 1)
                w = {j: r ** (d - j) for j in range(0, d + 1)}
            else:
                # keys 0..Skv-1 at distances |d - j|: those left of or on the diagonal and those right of it
                right = Skv - 1 - d
                z = r ** (d - left) * geo(left + 1) + (r * geo(right) if right > 0 else 0.0)
                w = {j: r ** abs(d - j) for j in range(Skv)}
            np.testing.assert_allclose(L[0, h, i], math.log(z), rtol=1e-13, atol=1e-13)
            ref_o = sum(wj * v[0, h, j] for j, wj in w.items()) / sum(w.values())
            np.testing.assert_allclose(O[0, h, i], ref_o, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(Ot[0, h, i], ref_o, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(Lt[0, h, i], math.log(z), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Sq,Skv,causal,window", MASK_CASES)
def test_dkdv_keys_against_torch_fp64(Sq, Skv, causal, window):
    """dK, dV of chosen keys (each summed over the rows that see it) against PyTorch's
    fp64 gradients of the masked attention."""
    r = np.random.default_rng(Sq * 7 + Skv)
    q = r.standard_normal((2, 4, Sq, 8)) * 1.5
    k, v = r.standard_normal((2, 2, Skv, 8)), r.standard_normal((2, 2, Skv, 8))
    do = r.standard_normal((2, 4, Sq, 8))
    vis, _, _, dk, dv = _torch_masked(q, k, v, do, 0.4, causal, window)
    do0 = np.where(vis.any(axis=1)[None, None, :, None], do, 0.0)
    keys = np.unique(np.concatenate([[0, Skv - 1], r.integers(0, Skv, 4)]))
    for b, g in ((0, 0), (1, 1)):
        gk, gv = oracle.sdpa_dkdv_keys(q, k, v, do0, 0.4, causal, b, g, keys, window=window)
        np.testing.assert_allclose(gk, dk[b, g, keys], atol=1e-12)
        np.testing.assert_allclose(gv, dv[b, g, keys], atol=1e-12)


def _torch_alibi(q, k, v, do, scale, causal, window, slopes):
    """PyTorch's fp64 SDPA with the bias passed as an additive float mask (-inf where hidden)."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off = Skv - Sq
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    vis = np.ones((Sq, Skv), dtype=bool)
    if causal:
        vis &= j <= i + off
    if window is not None:
        vis &= j >= i + off - window
    bias = np.stack([np.where(vis, -a * np.abs(i + off - j), -np.inf) for a in slopes])[None]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1),
                                         attn_mask=torch.tensor(bias), scale=scale)
    out.backward(torch.tensor(do))
    return {"o": out.detach().numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}


ALIBI_CASES = [(19, 19, True, None), (19, 19, False, None), (11, 23, True, 5), (23, 11, False, 3), (16, 16, True, 0)]


def test_dkdv_keys_alibi_against_torch_fp64():
    rng = np.random.default_rng(77)
    q = rng.standard_normal((2, 4, 21, 8)) * 1.5
    k, v = rng.standard_normal((2, 2, 21, 8)), rng.standard_normal((2, 2, 21, 8))
    do = rng.standard_normal((2, 4, 21, 8))
    ref = _torch_alibi(q, k, v, do, 0.35, True, None, SLOPES4)
    keys = np.array([0, 3, 10, 20])
    for b, g in ((0, 1), (1, 0)):
        gk, gv = oracle.sdpa_dkdv_keys(q, k, v, do, 0.35, True, b, g, keys, alibi=SLOPES4)
        np.testing.assert_allclose(gk, ref["dk"][b, g, keys], atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(gv, ref["dv"][b, g, keys], atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("Sq,Skv,causal,window", ALIBI_CASES)
def test_alibi_against_torch_fp64(Sq, Skv, causal, window):
    rng = np.random.default_rng(42 + Sq)
    q = rng.standard_normal((2, 4, Sq, 8)) * 1.5
    k = rng.standard_normal((2, 2, Skv, 8))
    v = rng.standard_normal((2, 2, Skv, 8))
    do = rng.standard_normal((2, 4, Sq, 8))
    if causal and Skv < Sq:
        pytest.skip("rows without keys have no softmax in torch")
    ref = _torch_alibi(q, k, v, do, 0.35, causal, window, SLOPES4)
    got = oracle.sdpa_backward(q, k, v, do, 0.35, causal, window=window, alibi=SLOPES4)
    for n in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(got[n], ref[n], atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("Sq,Skv,causal,window", ALIBI_CASES)
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 3), (16, 8)])
def test_alibi_tiled_equals_dense(Sq, Skv, causal, window, br, bc):
    rng = np.random.default_rng(43 + Skv)
    q = rng.standard_normal((1, 4, Sq, 4)) * 2
    k = rng.standard_normal((1, 2, Skv, 4))
    v = rng.standard_normal((1, 2, Skv, 4))
    do = rng.standard_normal((1, 4, Sq, 4))
    g = oracle.sdpa_backward(q, k, v, do, 0.6, causal, window=window, alibi=SLOPES4)
    O, L = oracle.online_forward(q, k, v, 0.6, causal, br, bc, window=window, alibi=SLOPES4)
    fin = np.isfinite(g["lse"])
    np.testing.assert_allclose(O, g["o"], atol=1e-12)
    np.testing.assert_allclose(L[fin], g["lse"][fin], atol=1e-12)
    dq, dk, dv = oracle.online_backward(q, k, v, O, L, do, 0.6, causal, br, bc, window=window, alibi=SLOPES4)
    np.testing.assert_allclose(dq, g["dq"], atol=1e-12)
    np.testing.assert_allclose(dk, g["dk"], atol=1e-12)
    np.testing.assert_allclose(dv, g["dv"], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_alibi_finite_differences(causal):
    q, k, v, do = rand_qkvdo(1, 4, 2, 9, 4, seed=44)
    scale = 0.5

    def f(q_, k_, v_):
        return float((oracle.sdpa_forward(q_, k_, v_, scale, causal, alibi=SLOPES4)[0] * do).sum())

    g = oracle.sdpa_backward(q, k, v, do, scale, causal, alibi=SLOPES4)
    h = 1e-6
    rng = np.random.default_rng(45)
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(10):
            ix = tuple(rng.integers(0, n) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[ix] += h
            minus[ix] -= h
            args_p = {"dq": (plus, k, v), "dk": (q, plus, v), "dv": (q, k, plus)}[name]
            args_m = {"dq": (minus, k, v), "dk": (q, minus, v), "dv": (q, k, minus)}[name]
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(g[name][ix] - fd) <= 1e-7 * max(1.0, abs(fd)), (name, ix, g[name][ix], fd)
