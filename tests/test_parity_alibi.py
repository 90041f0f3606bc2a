"""GPU parity of the linear position bias (ALiBi) against the fp64 CPU oracle.

Reading (the SDPA page only lists ALiBi in its support matrix): query i and key
j of query head h get -a_h * |i + offset - j| added to their scaled score, with
one slope per query head passed as a device vector.  Slopes are the common
geometric sequence 2^(-8(h+1)/Hq) (strong bias, most weight near the diagonal)
or a small one (every key counts).  Tolerances are those of ``test_parity``;
fp32 cases take the small slopes, since far keys under the strong ones put |L|
near 100, where the fp32 value itself rounds by up to 3.8e-6.
"""
import math

import numpy as np
import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import make_inputs, make_varlen_inputs

from test_parity import TOL, check_grads, check_o, dev, host, say
from test_parity_ex import check_lse, compare

pytestmark = pytest.mark.gpu


def geometric_slopes(Hq):
    return np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=np.float32)


def small_slopes(Hq):
    return np.array([1e-3 * (h + 1) for h in range(Hq)], dtype=np.float32)


def run(inp, dtype, scale, causal, window, slopes):
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    a = torch.from_numpy(slopes).to("cuda:0")
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal, window=window, alibi=a)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=scale, causal=causal, window=window, alibi=a)
    torch.cuda.synchronize()
    return host(o), host(lse), (host(dq), host(dk), host(dv))


CASES = []
for S, Skv in ((1, 1), (63, 63), (200, 200), (129, 333), (333, 129)):
    for D in (64, 128):
        for dtype in ("f32", "f16", "bf16"):
            for causal in (True, False):
                CASES.append((S, Skv, D, dtype, causal))


@pytest.mark.parametrize("Sq,Skv,D,dtype,causal", CASES)
def test_alibi_small(Sq, Skv, D, dtype, causal):
    G = (1, 2, 4)[(Sq + D) % 3]
    B, Hkv = 2, 2
    Hq = Hkv * G
    scale = 1.0 / math.sqrt(D)
    # fp32 takes the small slopes: with the strong ones the far keys put |L| near 100,
    # where one fp32 ulp (7.6e-6) is most of the literal 1e-5 gate; 16-bit types take both
    slopes = geometric_slopes(Hq) if (Sq + D) % 2 and dtype != "f32" else small_slopes(Hq)
    inp = make_inputs(B, Hq, Hkv, Sq, D, dtype, seed=5000 + Sq + Skv + D, q_std=1.5, Skv=Skv)
    what = f"alibi Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} G={G}"
    say("case", what)
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, alibi=slopes)
    compare(run(inp, dtype, scale, causal, None, slopes), ref, dtype, what)


@pytest.mark.parametrize("window,causal,dtype,D", [(40, True, "bf16", 128), (40, False, "f16", 64),
                                                    (0, True, "f32", 64), (150, True, "bf16", 64)])
def test_alibi_window(window, causal, dtype, D):
    Sq, Skv, Hq, Hkv = 300, 300, 4, 2
    scale = 1.0 / math.sqrt(D)
    slopes = small_slopes(Hq) if dtype == "f32" else geometric_slopes(Hq)
    inp = make_inputs(1, Hq, Hkv, Sq, D, dtype, seed=5100 + window, q_std=1.5, Skv=Skv)
    what = f"alibi window={window} causal={causal} {dtype} D={D}"
    say("case", what)
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, window=window, alibi=slopes)
    compare(run(inp, dtype, scale, causal, window, slopes), ref, dtype, what)


def test_alibi_varlen():
    sq = (7, 1, 100, 64, 200, 0)
    sk = (17, 1, 40, 64, 260, 5)
    Hq, Hkv, D, dtype = 4, 2, 128, "bf16"
    scale = 1.0 / math.sqrt(D)
    slopes = geometric_slopes(Hq)
    inp = make_varlen_inputs(sq, sk, Hq, Hkv, D, dtype, seed=5200, q_std=1.5)
    say("case alibi varlen")
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    cu_q = torch.from_numpy(inp["cu_q"]).to("cuda:0")
    cu_k = torch.from_numpy(inp["cu_k"]).to("cuda:0")
    a = torch.from_numpy(slopes).to("cuda:0")
    o, lse = fa.forward_varlen(q, k, v, cu_q, cu_k, max(sq), max(sk), scale=scale, causal=True, alibi=a)
    g = fa.backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, max(sq), max(sk), scale=scale, causal=True, alibi=a)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_varlen(inp["q"], inp["k"], inp["v"], inp["do"], inp["cu_q"], inp["cu_k"], scale,
                                      True, alibi=slopes)
    compare((host(o), host(lse), tuple(host(t) for t in g)), ref, dtype, "alibi varlen")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal,window,slopes", [(True, None, "geo"), (True, None, "small"),
                                                   (False, 300, "geo")])
def test_alibi_wide_grid(dtype, causal, window, slopes):
    """B = 8, 32/8 heads, S = 1999, D = 128: the 8-wave forward and dQ kernels with the
    bias; sampled rows of every eighth head and one whole KV group's gradients."""
    B, Hq, Hkv, S, D = 8, 32, 8, 1999, 128
    scale = 1.0 / math.sqrt(D)
    sl = geometric_slopes(Hq) if slopes == "geo" else small_slopes(Hq)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=5300 + (window or 0), q_std=2.0)
    what = f"alibi wide grid {dtype} causal={causal} window={window} slopes={slopes}"
    say("case", what)
    o, lse, (dq, dk, dv) = run(inp, dtype, scale, causal, window, sl)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, S - 1], rng.integers(0, S, 5)]))
    for b in (0, 7):
        for h in range(0, Hq, 8):
            Or, Lr = oracle.sdpa_forward_rows(inp["q"], inp["k"], inp["v"], scale, causal, b, h, rows,
                                              window=window, alibi=sl)
            check_o(o[b, h, rows], Or, dtype, f"{what} b={b} h={h}")
            check_lse(lse[b, h, rows], Lr, dtype, f"{what} b={b} h={h}")
    g = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, groups=[(3, 5)],
                             window=window, alibi=sl)
    heads = list(range(20, 24))
    check_o(o[3, heads], g["o"][3, heads], dtype, what + " group")
    check_grads((dq[3, heads], dk[3, 5], dv[3, 5]), (g["dq"][3, heads], g["dk"][3, 5], g["dv"][3, 5]), dtype, what)


def test_alibi_zero_slopes():
    """All slopes 0: the biased kernels compute c s + 0 first and then exponentiate
    s - m instead of c s - m; every output still meets the oracle, and O and L agree with
    the unbiased call within the dtype's rounding."""
    B, Hq, Hkv, S, D = 2, 4, 2, 257, 128
    inp = make_inputs(B, Hq, Hkv, S, D, "bf16", seed=5400)
    scale = 1.0 / math.sqrt(D)
    say("case alibi zero slopes")
    got = run(inp, "bf16", scale, True, None, np.zeros(Hq, dtype=np.float32))
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, True)
    compare(got, ref, "bf16", "alibi zero slopes")
