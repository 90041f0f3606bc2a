"""GPU parity of the split-KV decode path (fa_fwd_splitkv) against the fp64 oracle.

The oracle is the plain definition (``oracle.sdpa_forward`` with a longer key
sequence, diagonal aligned bottom-right; ``sdpa_forward_varlen`` for packed
batches): the split and its logsumexp merge must reproduce it to the forward's
tolerances.  Split counts cover 1, several, more ranges than key tiles (capped)
and the library's own choice; windows make most ranges empty (L_s = -inf).
"""
import math

import numpy as np
import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import DECODE, decode_inputs, make_inputs, make_varlen_inputs

from test_parity import TOL, check_o, dev, host, say
from test_parity_ex import check_lse

pytestmark = pytest.mark.gpu


def run_split(inp, dtype, scale, causal, window, num_splits):
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = fa.forward_splitkv(q, k, v, scale=scale, causal=causal, window=window, num_splits=num_splits)
    torch.cuda.synchronize()
    return host(o), host(lse)


CASES = []
for n, (Sq, Skv) in enumerate(((1, 1), (1, 37), (1, 300), (1, 2500), (3, 2), (3, 301), (8, 1000), (8, 5))):
    for D in (64, 128):
        for dtype in ("f32", "bf16", "f16"):
            causal = (n + D // 64 + len(dtype)) % 4 != 0
            window = (None, None, 100, 7)[(n + len(dtype)) % 4]
            splits = (0, 1, 5, 1000)[(n + D) % 4]
            CASES.append((Sq, Skv, D, dtype, causal, window, splits))


@pytest.mark.parametrize("Sq,Skv,D,dtype,causal,window,splits", CASES)
def test_decode_dense(Sq, Skv, D, dtype, causal, window, splits):
    B, Hkv, G = 3, 2, 4
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hkv * G, Hkv, Sq, D, dtype, seed=6000 + Sq * 7 + Skv, q_std=1.5, backward=False, Skv=Skv)
    what = f"decode Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} window={window} splits={splits}"
    say("case", what)
    O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], scale, causal, window=window)
    o, lse = run_split(inp, dtype, scale, causal, window, splits)
    check_o(o, O, dtype, what)
    check_lse(lse, L, dtype, what)


@pytest.mark.parametrize("G,Sq", [(1, 32), (8, 4), (32, 1), (2, 16)])
def test_decode_full_row_block(G, Sq):
    """(Hq / Hkv) * Sq = 32: the group's rows fill the whole 32-column block."""
    B, Hkv, Skv, D = 2, 2, 777, 128
    inp = make_inputs(B, Hkv * G, Hkv, Sq, D, "bf16", seed=6100 + G, q_std=2.0, backward=False, Skv=Skv)
    say(f"case G={G} Sq={Sq}")
    O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], 1 / math.sqrt(D), True)
    o, lse = run_split(inp, "bf16", 1 / math.sqrt(D), True, None, 0)
    check_o(o, O, "bf16", f"G={G} Sq={Sq}")
    check_lse(lse, L, "bf16", f"G={G} Sq={Sq}")


def test_decode_no_keys_and_short_caches():
    """Skv = 0: every row is empty.  Skv < Sq, causal: the first Sq - Skv rows are empty."""
    say("case decode Skv=0 / Skv<Sq")
    inp = make_inputs(2, 4, 2, 4, 64, "bf16", seed=6200, backward=False, Skv=0)
    o, lse = run_split(inp, "bf16", 0.125, True, None, 0)
    assert not o.any() and np.isneginf(lse).all()
    inp = make_inputs(2, 4, 2, 6, 64, "bf16", seed=6201, backward=False, Skv=3)
    O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], 0.125, True)
    o, lse = run_split(inp, "bf16", 0.125, True, None, 3)
    check_o(o, O, "bf16")
    check_lse(lse, L, "bf16")


@pytest.mark.parametrize("causal,window,dtype", [(True, None, "bf16"), (False, None, "f32"), (True, 50, "f16")])
def test_decode_packed(causal, window, dtype):
    """Packed batch of single-token queries against caches of mixed lengths (some empty)."""
    sk = (0, 1, 100, 5000, 130, 64, 2049)
    sq = tuple(1 if n > 0 else 0 for n in sk)[:-1] + (2,)
    Hq, Hkv, D = 8, 2, 128
    inp = make_varlen_inputs(sq, sk, Hq, Hkv, D, dtype, seed=6300, q_std=1.5)
    say(f"case decode packed causal={causal} window={window} {dtype}")
    O, L = oracle.sdpa_forward_varlen(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 1 / math.sqrt(D),
                                      causal, window)
    q, k, v = (dev(inp[n], dtype) for n in ("q", "k", "v"))
    cu_q = torch.from_numpy(inp["cu_q"]).to("cuda:0")
    cu_k = torch.from_numpy(inp["cu_k"]).to("cuda:0")
    o, lse = fa.forward_splitkv(q, k, v, causal=causal, window=window, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                                max_seqlen_q=max(sq), max_seqlen_k=max(sk))
    torch.cuda.synchronize()
    check_o(host(o), O, dtype, "packed decode")
    check_lse(host(lse), L, dtype, "packed decode")


def test_decode_workload_full_size():
    """The decode workload at full size (16 sequences x 8192 cached keys, 32/8 heads,
    D = 128, bf16): every row against the oracle, the non-split forward agrees, and
    two calls are bitwise equal."""
    w = DECODE
    inp = decode_inputs(w)
    say(f"workload {w.name}")
    O, L = oracle.sdpa_forward(inp["q"], inp["k"], inp["v"], w.scale, True)
    q, k, v = (dev(inp[n], w.dtype) for n in ("q", "k", "v"))
    o1, l1 = fa.forward_splitkv(q, k, v, scale=w.scale)
    o2, l2 = fa.forward_splitkv(q, k, v, scale=w.scale)
    o3, l3 = fa.forward(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    eo = check_o(host(o1), O, w.dtype, w.name)
    check_lse(host(l1), L, w.dtype, w.name)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check_o(host(o3), O, w.dtype, w.name + " (non-split)")
    say(f"  O max-abs {eo:.3e}, L max-abs {float(np.abs(host(l1) - L).max()):.3e}")
