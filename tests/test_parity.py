"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Both sides read the same seeded, dtype-rounded inputs (``workloads``).
Tolerances (stated for this attention target): fp32 inputs -- O and L within
max-abs 1e-5, gradients within rel-L2 1e-4; bf16 / fp16 inputs -- O within
max-abs 1e-2, L within max-abs 1e-2, gradients within rel-L2 2e-2.

bf16 storage caveat: a bf16 output cannot be closer to the exact value than
half a bf16 ulp.  bf16 keeps 8 significant bits, so half an ulp is 2^-7 = 0.0078
for |O| in [2, 4), below the gate, and 2^-6 = 0.0156 for |O| in [4, 8), above
it.  The O gate is the literal max-abs 1e-2; an element above it is accepted
only where |O_ref| >= 4 (where storing it in bf16 alone can cost more than
1e-2) and the error is at most one bf16 ulp of O_ref, and every such
acceptance is printed.
"""
import math
import sys

import numpy as np
import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {
    "f32": dict(o=1e-5, lse=1e-5, grad=1e-4),
    "f16": dict(o=1e-2, lse=1e-2, grad=2e-2),
    "bf16": dict(o=1e-2, lse=1e-2, grad=2e-2),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(TORCH_DTYPE[dtype]).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_forward(inp, dtype, scale, causal):
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


def gpu_backward(tensors, o, lse, do_np, dtype, scale, causal):
    q, k, v = tensors
    do = dev(do_np, dtype)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - 7)


def check_o(got, ref, dtype, what=""):
    err = np.abs(got - ref)
    tol = TOL[dtype]["o"]
    bad = err > tol
    if bad.any():
        assert dtype == "bf16", f"{what} O max-abs {err.max():.3e} > {tol}"
        ok = (np.abs(ref[bad]) >= 4.0) & (err[bad] <= bf16_ulp(ref[bad]))
        assert ok.all(), f"{what} O max-abs {err.max():.3e} > {tol} at |O_ref| < 4 or beyond 1 ulp"
        say(f"  {what}: {int(bad.sum())} O elements over {tol} (max {err.max():.4f}), all at |O_ref| >= 4 "
            f"within one bf16 ulp: pass under the storage-rounding reading")
    return float(err.max())


def rel_l2(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def check_grads(got, ref, dtype, what=""):
    """rel-L2 per gradient.  Where the exact gradient is identically zero (S = 1, say)
    the ratio is undefined; there the GPU values, pure rounding residue, must stay
    below the same bound in absolute terms (inputs are O(1))."""
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        if not np.any(r):
            e = float(np.abs(g).max())
            assert e <= TOL[dtype]["grad"], f"{what} {name}: exact value is 0, GPU max-abs {e:.3e}"
        else:
            e = rel_l2(g, r)
            assert e <= TOL[dtype]["grad"], f"{what} {name} rel-L2 {e:.3e} > {TOL[dtype]['grad']}"
        out[name] = e
    return out


# ------------------------------------------------------------------ small ragged sweep

SWEEP = []
for S in (1, 2, 63, 65, 127, 129, 200):
    for D in (64, 128):
        for dtype in ("f32", "f16", "bf16"):
            for causal in (True, False):
                G = (1, 2, 4)[(S + D // 64 + len(dtype)) % 3]
                SWEEP.append((S, D, dtype, causal, G))


@pytest.mark.parametrize("S,D,dtype,causal,G", SWEEP)
def test_small_sweep(S, D, dtype, causal, G):
    B, Hkv = 2, 2
    Hq = Hkv * G
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=1000 + S + D, q_std=1.5)
    say(f"case S={S} D={D} {dtype} causal={causal} G={G}")
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    t, o, lse = gpu_forward(inp, dtype, scale, causal)
    check_o(host(o), ref["o"], dtype)
    assert np.abs(host(lse) - ref["lse"]).max() <= TOL[dtype]["lse"]
    got = gpu_backward(t, o, lse, inp["do"], dtype, scale, causal)
    check_grads(got, (ref["dq"], ref["dk"], ref["dv"]), dtype)


# ------------------------------------------------------------------ the five workloads

def _full_check(w):
    inp = workload_inputs(w)
    say(f"workload {w.name}")
    t, o, lse = gpu_forward(inp, w.dtype, w.scale, w.causal)
    if w.backward:
        ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, w.causal)
    else:
        O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
        ref = {"o": O, "lse": L}
    eo = check_o(host(o), ref["o"], w.dtype, w.name)
    el = float(np.abs(host(lse) - ref["lse"]).max())
    assert el <= TOL[w.dtype]["lse"], el
    msg = f"  {w.name}: O max-abs {eo:.3e}, L max-abs {el:.3e}"
    if w.backward:
        got = gpu_backward(t, o, lse, inp["do"], w.dtype, w.scale, w.causal)
        g = check_grads(got, (ref["dq"], ref["dk"], ref["dv"]), w.dtype, w.name)
        msg += ", rel-L2 " + ", ".join(f"{k} {v:.3e}" for k, v in g.items())
    say(msg)


def test_workload_small_fp32():
    _full_check(WORKLOADS["causal_f32_b1_h2_s128_d64"])


def test_workload_gpt2_small_bf16():
    _full_check(WORKLOADS["gpt2s_causal_bf16_b8_h12_s1024_d64"])


def test_workload_qwen3_gqa_bf16_forward():
    _full_check(WORKLOADS["qwen3_gqa_causal_bf16_b4_h32kv8_s2048_d128"])


def test_workload_fp16_s4096():
    _full_check(WORKLOADS["causal_f16_b1_h8_s4096_d64"])


def test_workload_long_context_gqa_bf16():
    """S = 16384: one whole KV group (4 query heads, every row) fwd + bwd; in every head, O and L of
    every 8th row and dQ of every 64th (the first row varies with the head, so across the heads every
    row position modulo 8 is checked), with the tile-edge rows; dK, dV of the last keys of every KV
    group."""
    w = WORKLOADS["longctx_gqa_causal_bf16_b1_h32kv8_s16384_d128"]
    inp = workload_inputs(w)
    say(f"workload {w.name}")
    t, o, lse = gpu_forward(inp, w.dtype, w.scale, w.causal)
    O, L = host(o), host(lse)
    got = gpu_backward(t, o, lse, inp["do"], w.dtype, w.scale, w.causal)
    g = w.Hkv - 1
    heads = list(range(g * w.group, (g + 1) * w.group))
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, True, groups=[(0, g)])
    eo = check_o(O[0, heads], ref["o"][0, heads], w.dtype, w.name + " group")
    el = float(np.abs(L[0, heads] - ref["lse"][0, heads]).max())
    assert el <= TOL[w.dtype]["lse"]
    e = check_grads((got[0][0, heads], got[1][0, g], got[2][0, g]),
                    (ref["dq"][0, heads], ref["dk"][0, g], ref["dv"][0, g]), w.dtype, w.name)
    say(f"  group {g}: O max-abs {eo:.3e}, L {el:.3e}, " + ", ".join(f"{k} {v:.3e}" for k, v in e.items()))
    rng = np.random.default_rng(7)
    edge = np.array([0, 1, 127, 128, 255, 256, w.S - 2, w.S - 1])
    worst_o = worst_l = 0.0
    n_o = 0
    dq_got, dq_ref = [], []
    for h in range(w.Hq):
        rows = np.union1d(np.arange(h % 8, w.S, 8), edge)
        n_o += rows.size
        for c in range(0, rows.size, 512):
            rc = rows[c:c + 512]
            Or, Lr = oracle.sdpa_forward_rows(inp["q"], inp["k"], inp["v"], w.scale, True, 0, h, rc)
            worst_o = max(worst_o, check_o(O[0, h, rc], Or, w.dtype, f"head {h} rows"))
            worst_l = max(worst_l, float(np.abs(L[0, h, rc] - Lr).max()))
        rows = np.union1d(np.arange(h % 64, w.S, 64), edge)
        dq_ref.append(oracle.sdpa_dq_rows(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, True, 0, h, rows))
        dq_got.append(got[0][0, h, rows])
    assert worst_l <= TOL[w.dtype]["lse"], worst_l
    e = rel_l2(np.concatenate(dq_got), np.concatenate(dq_ref))
    assert e <= TOL[w.dtype]["grad"], e
    say(f"  {n_o} O rows of all heads: O max-abs {worst_o:.3e}, L {worst_l:.3e}; "
        f"{sum(len(x) for x in dq_got)} dQ rows: rel-L2 {e:.3e}")
    # dK, dV of the last keys of every KV group (seen by the last rows only, so the
    # oracle forms 256 rows per head): the groups the whole-group check leaves out
    keys = np.unique(np.concatenate([np.arange(w.S - 32, w.S), rng.integers(w.S - 256, w.S, 8)]))
    dkg, dkr, dvg, dvr = [], [], [], []
    for g2 in range(w.Hkv):
        rk, rv = oracle.sdpa_dkdv_keys(inp["q"], inp["k"], inp["v"], inp["do"], w.scale, True, 0, g2, keys)
        dkg.append(got[1][0, g2, keys]), dkr.append(rk), dvg.append(got[2][0, g2, keys]), dvr.append(rv)
    ek, ev = rel_l2(np.stack(dkg), np.stack(dkr)), rel_l2(np.stack(dvg), np.stack(dvr))
    assert ek <= TOL[w.dtype]["grad"] and ev <= TOL[w.dtype]["grad"], (ek, ev)
    say(f"  last keys of all KV groups: dk rel-L2 {ek:.3e}, dv rel-L2 {ev:.3e}")


# ------------------------------------------------------------------ closed forms and edge cases

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_row0_and_single_position_exact(dtype, D):
    inp = make_inputs(1, 4, 2, 300, D, dtype, seed=5)
    _, o, lse = gpu_forward(inp, dtype, 1.0 / math.sqrt(D), True)
    O = host(o)
    v = inp["v"].astype(np.float64)
    # Row 0 sees only key 0: O = V[0].  bf16 / fp16 give it bit-exactly (P rounds to 1);
    # fp32 keeps p = exp2(s*c - round(s*c)), within 1e-7 of 1, so O is within 1 ulp.
    rtol = 0 if dtype != "f32" else 2.0 ** -22
    np.testing.assert_allclose(O[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0), rtol=rtol, atol=0)
    one = make_inputs(2, 4, 4, 1, D, dtype, seed=6)
    t, o1, l1 = gpu_forward(one, dtype, 0.1, True)
    np.testing.assert_allclose(host(o1), one["v"].astype(np.float64), rtol=rtol, atol=0)
    dq, dk, dv = gpu_backward(t, o1, l1, one["do"], dtype, 0.1, True)
    # dS = P (dP - D) with P = 1 and dP = D mathematically: only rounding residue remains
    assert np.abs(dq).max() <= 1e-4 and np.abs(dk).max() <= 1e-4
    # dV = P^T dO with P = exp(s - L) = 1 up to the rounding of the stored L
    np.testing.assert_allclose(dv, one["do"].astype(np.float64), rtol=2e-6, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_queries_give_prefix_means(dtype):
    S, D = 333, 64
    inp = make_inputs(1, 2, 1, S, D, dtype, seed=9)
    inp["q"][:] = 0
    t, o, lse = gpu_forward(inp, dtype, 0.125, True)
    i = np.arange(S)
    mean_v = np.cumsum(inp["v"].astype(np.float64), axis=2) / (i + 1)[None, None, :, None]
    check_o(host(o), np.repeat(mean_v, 2, axis=1), dtype)
    np.testing.assert_allclose(host(lse)[0, 0], np.log(i + 1.0), atol=TOL[dtype]["lse"])
    _, dk, _ = gpu_backward(t, o, lse, inp["do"], dtype, 0.125, True)
    assert np.abs(dk).max() <= 1e-6            # Q = 0 gives dK = 0 up to rounding of P


def test_empty_problem_is_a_noop():
    q = torch.empty(0, 2, 16, 64, device="cuda:0", dtype=torch.bfloat16)
    o, lse = fa.forward(q, q[:, :1], q[:, :1])
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


def test_large_ragged_sequence():
    S, D = 3001, 128
    inp = make_inputs(1, 4, 1, S, D, "bf16", seed=21)
    scale = 1.0 / math.sqrt(D)
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    t, o, lse = gpu_forward(inp, "bf16", scale, True)
    check_o(host(o), ref["o"], "bf16")
    assert np.abs(host(lse) - ref["lse"]).max() <= 1e-2
    got = gpu_backward(t, o, lse, inp["do"], "bf16", scale, True)
    check_grads(got, (ref["dq"], ref["dk"], ref["dv"]), "bf16")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_repeat_determinism(dtype):
    inp = make_inputs(2, 8, 2, 777, 128, dtype, seed=31)
    a = gpu_forward(inp, dtype, 0.09, True)
    b = gpu_forward(inp, dtype, 0.09, True)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    ga = gpu_backward(a[0], a[1], a[2], inp["do"], dtype, 0.09, True)
    gb = gpu_backward(a[0], a[1], a[2], inp["do"], dtype, 0.09, True)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


# ------------------------------------------------------------------ closed forms on the 8-wave path

# B = 8, 32 query heads over 8 KV heads, S = 1999, D = 128: ceil(1999 / 256) * 8 * 32 =
# 2048 eight-wave query blocks, so both the forward (8 waves from 256 blocks at D = 128)
# and dQ (8 waves from 2048 blocks) take their 8-wave kernels; 1999 keys end inside a
# 128-key load stage.
WIDE8 = dict(B=8, Hq=32, Hkv=8, S=1999, D=128)


def _group_oracle(inp, scale, b, g):
    """The oracle's fwd + bwd of one whole KV group (all of its query heads and rows)."""
    return oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True, groups=[(b, g)])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_constant_values_closed_form(dtype):
    """Every key of a KV head carries the same value row c (P3).  Then O = c for every
    query whatever the weights, and dQ = dK = 0: dP_ij = dO_i . c = D_i for every key, so
    dS = P (dP - D) vanishes.  On the GPU O equals c bit for bit (the weight sums of
    P V and of l agree to fp32 rounding, far inside half an ulp of the dtype), dQ and dK
    are pure rounding residue, and dV = P^T dO meets the oracle."""
    w = WIDE8
    G = w["Hq"] // w["Hkv"]
    scale = 1.0 / math.sqrt(w["D"])
    inp = make_inputs(w["B"], w["Hq"], w["Hkv"], w["S"], w["D"], dtype, seed=41, q_std=2.0)
    inp["v"][:] = inp["v"][:, :, :1, :]
    say(f"case constant V {dtype} {w}")
    t, o, lse = gpu_forward(inp, dtype, scale, True)
    O = host(o)
    c = np.repeat(inp["v"][:, :, :1, :].astype(np.float64), G, axis=1)
    assert np.array_equal(O, np.broadcast_to(c, O.shape)), "O != c"
    dq, dk, dv = gpu_backward(t, o, lse, inp["do"], dtype, scale, True)
    eq, ek = float(np.abs(dq).max()), float(np.abs(dk).max())
    say(f"  max |dQ| {eq:.2e}, max |dK| {ek:.2e}")
    assert eq <= 1e-3 and ek <= 1e-3
    b, g = 5, 3
    ref = _group_oracle(inp, scale, b, g)
    e = rel_l2(dv[b, g], ref["dv"][b, g])
    assert e <= TOL[dtype]["grad"], f"dV rel-L2 {e:.3e}"
    assert np.abs(ref["dq"][b, g * G:(g + 1) * G]).max() <= 1e-12  # the oracle agrees: dQ = 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_key_shift_closed_form(dtype):
    """Adding one vector u to every key of a KV head moves each query row's scores by the
    constant scale * q_i . u (P5): the softmax weights do not change, so O, dQ and dK do
    not, while L moves by exactly scale * q_i . u.

    Keys are drawn on a 1/16 grid inside (-8, 8) and every element of u is +-2 or +-8,
    so K + u is exact in bf16 and fp16 (at most 8 significant bits) and both runs see
    the intended inputs.  With u = +-8 the shifts reach tens of natural-log units, which
    moves the forward's running reference far from the first tile's.  Each run is held
    to the same oracle (the unshifted problem's O, dQ, dK; its L plus the shift).  The
    backward is checked with u = +-2: dQ of the shifted keys adds scale * u * sum_j dS_ij,
    zero exactly but not after dS is rounded to the dtype, and that residue grows with |u|."""
    w = WIDE8
    B, Hq, Hkv, S, D = w["B"], w["Hq"], w["Hkv"], w["S"], w["D"]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=43, q_std=2.0)
    inp["k"] = np.clip(np.round(inp["k"] * 16) / 16, -127 / 16, 127 / 16).astype(np.float32)
    sign = np.where(np.random.default_rng(44).random(D) < 0.5, -1.0, 1.0)
    b, g = 6, 2
    heads = list(range(g * G, (g + 1) * G))
    ref = _group_oracle(inp, scale, b, g)
    q64 = inp["q"].astype(np.float64)
    rng = np.random.default_rng(45)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, S - 1], rng.integers(0, S, 9)]))
    for mag in (8.0, 2.0):
        u = (mag * sign).astype(np.float32)
        shifted = dict(inp, k=(inp["k"] + u).astype(np.float32))
        # the shifted keys must be exact in the dtype, else the two problems differ
        from workloads import round_to
        assert np.array_equal(round_to(shifted["k"], dtype), shifted["k"])
        say(f"case key shift |u| = {mag} {dtype} {w}")
        t, o, lse = gpu_forward(shifted, dtype, scale, True)
        O, L = host(o), host(lse)
        shift = scale * np.einsum("bhsd,d->bhs", q64, u.astype(np.float64))
        check_o(O[b, heads], ref["o"][b, heads], dtype, f"|u|={mag} group")
        el = float(np.abs(L[b, heads] - (ref["lse"][b, heads] + shift[b, heads])).max())
        assert el <= TOL[dtype]["lse"], f"|u|={mag}: L max-abs {el:.3e} from L_ref + scale q.u"
        # sampled rows of every head: O unchanged, L shifted
        for h in range(0, Hq, 3):
            bb = h % B
            Or, Lr = oracle.sdpa_forward_rows(inp["q"], inp["k"], inp["v"], scale, True, bb, h, rows)
            check_o(O[bb, h, rows], Or, dtype, f"|u|={mag} b={bb} h={h}")
            e = float(np.abs(L[bb, h, rows] - (Lr + shift[bb, h, rows])).max())
            assert e <= TOL[dtype]["lse"], f"|u|={mag} b={bb} h={h}: L max-abs {e:.3e}"
        say(f"  |u|={mag}: group L max-abs {el:.3e} after the shift")
        if mag == 2.0:
            dq, dk, dv = gpu_backward(t, o, lse, inp["do"], dtype, scale, True)
            e = check_grads((dq[b, heads], dk[b, g], dv[b, g]),
                            (ref["dq"][b, heads], ref["dk"][b, g], ref["dv"][b, g]), dtype, f"|u|={mag}")
            say("  rel-L2 " + ", ".join(f"{k} {v:.3e}" for k, v in e.items()))
