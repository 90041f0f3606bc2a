"""fa_bwd_noalloc, the backward entry point that allocates nothing, against fa_bwd.

The row dot products live in the library's static device array instead of a
caller workspace; the kernels are the same, so every gradient must equal
fa_bwd's bit for bit.  Two calls in a row, the second on a smaller problem
(the array keeps the first call's contents), and a third on the first problem
again.  One of them is also held to the oracle.
"""
import math

import numpy as np
import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import make_inputs

from test_parity import TOL, check_grads, dev, host, say

pytestmark = pytest.mark.gpu

CODE = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}


def _run(B, Hq, Hkv, S, D, dtype, seed):
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=seed, q_std=1.5)
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale=scale, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, scale=scale, causal=True)   # fa_bwd with a workspace
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    s = torch.cuda.current_stream().cuda_stream
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           *(t.data_ptr() for t in got), B, Hq, Hkv, S, D, scale, True, CODE[dtype], s)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{name} of fa_bwd_noalloc differs from fa_bwd"
    return inp, scale, [host(t) for t in got]


def test_noalloc_backward_matches_workspace_backward():
    say("case noalloc bf16 B=2 Hq=32 Hkv=8 S=1500 D=128")
    inp, scale, got = _run(2, 32, 8, 1500, 128, "bf16", seed=61)
    say("case noalloc f16 B=1 Hq=4 Hkv=2 S=333 D=64 (smaller, after the larger)")
    inp2, scale2, got2 = _run(1, 4, 2, 333, 64, "f16", seed=62)
    ref = oracle.sdpa_backward(inp2["q"], inp2["k"], inp2["v"], inp2["do"], scale2, True)
    check_grads(got2, (ref["dq"], ref["dk"], ref["dv"]), "f16", "noalloc f16")
    say("case noalloc bf16 again, after the smaller call")
    _run(2, 32, 8, 1500, 128, "bf16", seed=63)


def test_noalloc_rejects_problems_beyond_the_array():
    rows = fa.FA_BWD_NOALLOC_MAX_ROWS
    A = 0x10000
    s = torch.cuda.current_stream().cuda_stream
    # B * Hq * S = rows + 64: one sequence too many for the array; rejected before any launch
    st = fa.fa_bwd_noalloc(A, A, A, A, A, A, A, A, A, 1, 64, 64, rows // 64 + 1, 64, 0.125, True, fa.FA_BF16, s)
    assert st == fa.FA_ERR_WORKSPACE
