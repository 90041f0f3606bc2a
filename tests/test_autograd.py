"""GPU: ``fa.attention`` as a torch autograd operation.

One forward and one ``backward()`` through torch's autograd, on small problems with
the causal, full, windowed and cross-length masks: O and the gradients of q, k and v
meet the fp64 oracle's bounds, and they are bit for bit the explicit ``fa.forward`` /
``fa.backward`` calls (the autograd node only connects the same kernels).
"""
import math

import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import make_inputs

from test_parity import check_grads, check_o, dev, host, say

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, causal, window, Skv (None: Skv = Sq)
    ("bf16", True, None, None),
    ("f32", True, None, None),
    ("f16", False, None, None),
    ("bf16", True, 40, None),
    ("bf16", True, None, 150),
]


@pytest.mark.parametrize("dtype,causal,window,Skv", CASES)
def test_autograd_matches_oracle_and_explicit_calls(dtype, causal, window, Skv):
    B, Hq, Hkv, S, D = 2, 4, 2, 100, 64
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=77 + (window or 0) + (Skv or 0), q_std=1.5, Skv=Skv)
    say(f"case autograd {dtype} causal={causal} window={window} Skv={Skv or S}")
    q, k, v = (dev(inp[n], dtype).requires_grad_() for n in ("q", "k", "v"))
    do = dev(inp["do"], dtype)
    o = fa.attention(q, k, v, scale=scale, causal=causal, window=window)
    o.backward(do)
    torch.cuda.synchronize()

    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, window=window)
    check_o(host(o.detach()), ref["o"], dtype, "autograd O")
    check_grads((host(q.grad), host(k.grad), host(v.grad)), (ref["dq"], ref["dk"], ref["dv"]), dtype, "autograd")

    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o2, lse2 = fa.forward(qd, kd, vd, scale=scale, causal=causal, window=window)
    grads = fa.backward(qd, kd, vd, o2, lse2, do, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for name, a, b in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), grads):
        assert torch.equal(a, b), f"autograd {name} differs from the explicit backward"
