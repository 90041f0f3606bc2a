"""GPU parity of the extended problems against the fp64 CPU oracle.

Covers queries and keys of different lengths (causal diagonal aligned
bottom-right), sliding windows, and packed variable-length batches, through
``fa_fwd_ex`` / ``fa_bwd_ex`` (and, for equal lengths without a window, the
plain entry points for comparison).  Tolerances are those of ``test_parity``.

Rows that see no key (a causal problem with fewer keys than queries, or a
sequence with no keys) have O = 0 and L = -inf on both sides; the -inf
positions must agree exactly and the finite L values meet the usual bound.
"""
import math

import numpy as np
import pytest
import torch

import causal_attention_fa_amd as fa
import oracle
from workloads import make_inputs, make_varlen_inputs

from test_parity import TOL, check_grads, check_o, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


def check_lse(got, ref, dtype, what=""):
    gi, ri = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"{what} L = -inf at different rows ({int(gi.sum())} vs {int(ri.sum())})"
    if (~ri).any():
        e = float(np.abs(got[~ri] - ref[~ri]).max())
        assert e <= TOL[dtype]["lse"], f"{what} L max-abs {e:.3e}"
    assert not np.isnan(got).any()


def run_dense(inp, dtype, scale, causal, window):
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal, window=window)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return host(o), host(lse), (host(dq), host(dk), host(dv))


def compare(got, ref, dtype, what):
    o, lse, grads = got
    check_o(o, ref["o"], dtype, what)
    check_lse(lse, ref["lse"], dtype, what)
    check_grads(grads, (ref["dq"], ref["dk"], ref["dv"]), dtype, what)


# ------------------------------------------------------------------ Sq != Skv

CROSS = []
for Sq, Skv in ((1, 257), (33, 200), (200, 33), (64, 81), (129, 65), (65, 1)):
    for D in (64, 128):
        for dtype in ("f32", "bf16"):
            for causal in (True, False):
                CROSS.append((Sq, Skv, D, dtype, causal))


@pytest.mark.parametrize("Sq,Skv,D,dtype,causal", CROSS)
def test_cross_length(Sq, Skv, D, dtype, causal):
    G = (1, 2, 4)[(Sq + Skv + D) % 3]
    B, Hkv = 2, 2
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hkv * G, Hkv, Sq, D, dtype, seed=2000 + Sq + 3 * Skv, q_std=1.5, Skv=Skv)
    what = f"Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} G={G}"
    say("case", what)
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal)
    compare(run_dense(inp, dtype, scale, causal, None), ref, dtype, what)


# ------------------------------------------------------------------ sliding window

WINDOWS = []
for Sq, Skv, win in ((300, 300, 0), (300, 300, 1), (300, 300, 31), (300, 300, 64), (300, 300, 100),
                     (257, 513, 40), (513, 257, 200), (130, 130, 1000)):
    for causal in (True, False):
        for dtype, D in (("bf16", 128), ("f32", 64), ("f16", 64)):
            WINDOWS.append((Sq, Skv, win, causal, dtype, D))


@pytest.mark.parametrize("Sq,Skv,window,causal,dtype,D", WINDOWS)
def test_window(Sq, Skv, window, causal, dtype, D):
    G = 2 if D == 128 else 1
    B, Hkv = 1, 2
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hkv * G, Hkv, Sq, D, dtype, seed=3000 + window + Sq, q_std=1.5, Skv=Skv)
    what = f"Sq={Sq} Skv={Skv} window={window} causal={causal} {dtype} D={D}"
    say("case", what)
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, window=window)
    compare(run_dense(inp, dtype, scale, causal, window), ref, dtype, what)


def test_no_keys_dense():
    """Skv = 0: every row's softmax is empty: O = 0, L = -inf, dQ = 0."""
    inp = make_inputs(1, 2, 1, 37, 64, "bf16", seed=7, Skv=0)
    say("case Skv=0")
    o, lse, (dq, dk, dv) = run_dense(inp, "bf16", 0.125, True, None)
    assert not o.any() and np.isneginf(lse).all() and not dq.any()
    assert dk.shape == (1, 1, 0, 64) and dv.shape == (1, 1, 0, 64)


def test_no_queries_dense():
    """Sq = 0 with keys: no query sees a key, so dK = dV = 0 (written, not left stale)."""
    Sq, Skv, D = 0, 100, 128
    q = torch.empty(1, 4, Sq, D, device="cuda:0", dtype=torch.bfloat16)
    k = torch.randn(1, 2, Skv, D, device="cuda:0").to(torch.bfloat16)
    v = torch.randn_like(k)
    say("case Sq=0")
    o, lse = fa.forward(q, k, v, window=5)
    dq, dk, dv = fa.backward(q, k, v, o, lse, torch.empty_like(q), window=5)
    torch.cuda.synchronize()
    assert o.shape == q.shape and dq.shape == q.shape
    assert not dk.float().abs().sum().item() and not dv.float().abs().sum().item()


# ------------------------------------------------------------------ packed variable-length batches

VARLEN = [
    # (query lengths, key lengths, causal, window, dtype, D)
    ((0, 1, 63, 64, 129, 300, 5), (0, 1, 63, 64, 129, 300, 5), True, None, "bf16", 128),
    ((0, 1, 63, 64, 129, 300, 5), (0, 1, 63, 64, 129, 300, 5), False, None, "f32", 64),
    ((7, 1, 100, 64, 200, 31, 5, 0), (17, 1, 40, 64, 65, 300, 0, 23), True, None, "bf16", 64),
    ((7, 1, 100, 64, 200, 31, 5, 0), (17, 1, 40, 64, 65, 300, 0, 23), False, None, "f16", 128),
    ((129, 300, 1, 64), (129, 300, 1, 64), True, 32, "bf16", 128),
    ((50, 300, 1, 64), (129, 200, 9, 64), True, 20, "f32", 128),
    ((50, 300, 1, 64), (129, 200, 9, 64), False, 70, "bf16", 64),
]


def run_varlen(inp, dtype, scale, causal, window, Hq):
    q, k, v, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    cu_q = torch.from_numpy(inp["cu_q"]).to("cuda:0")
    cu_k = torch.from_numpy(inp["cu_k"]).to("cuda:0")
    mq = int(np.diff(inp["cu_q"]).max())
    mk = int(np.diff(inp["cu_k"]).max())
    o, lse = fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, scale=scale, causal=causal, window=window)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, scale=scale, causal=causal,
                                    window=window)
    torch.cuda.synchronize()
    return host(o), host(lse), (host(dq), host(dk), host(dv))


@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen(case):
    sq, sk, causal, window, dtype, D = VARLEN[case]
    Hq, Hkv = 4, 2
    scale = 1.0 / math.sqrt(D)
    inp = make_varlen_inputs(sq, sk, Hq, Hkv, D, dtype, seed=4000 + case, q_std=1.5)
    what = f"varlen q={sq} k={sk} causal={causal} window={window} {dtype} D={D}"
    say("case", what)
    ref = oracle.sdpa_backward_varlen(inp["q"], inp["k"], inp["v"], inp["do"], inp["cu_q"], inp["cu_k"],
                                      scale, causal, window)
    compare(run_varlen(inp, dtype, scale, causal, window, Hq), ref, dtype, what)


def test_varlen_matches_dense_calls():
    """At full size (16401 packed tokens, 32 query / 8 KV heads, D = 128, bf16): every
    sequence of the packed call matches a dense call on that sequence alone.  Where the
    dense call runs the same kernels (8-wave forward tiles of 128 keys: 2048 tokens or
    more at 32 heads) the two agree bit for bit (dK, dV of a small dense grid to within
    one bf16 step: see below), which also rules out a single key
    leaking across a sequence boundary; shorter sequences run the 4-wave forward, whose
    64-key tiles round differently; there both calls meet the oracle's bounds.  Sampled
    rows of long and short sequences meet the oracle, and so do whole short sequences."""
    lens = (8192, 4096, 2048, 1024, 512, 256, 128, 64, 64, 17)
    Hq, Hkv, D, dtype = 32, 8, 128, "bf16"
    scale = 1.0 / math.sqrt(D)
    inp = make_varlen_inputs(lens, lens, Hq, Hkv, D, dtype, seed=4100, q_std=3.0)
    say("case varlen full size", lens)
    o, lse, (dq, dk, dv) = run_varlen(inp, dtype, scale, True, None, Hq)
    cu = inp["cu_q"]
    for b in (0, 2, 4, 9):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        sub = {n: np.ascontiguousarray(inp[n][None, :, r0:r1]) for n in ("q", "k", "v", "do")}
        do_, dl, (dq_, dk_, dv_) = run_dense(sub, dtype, scale, True, None)
        got = (o[:, r0:r1], lse[:, r0:r1], (dq[:, r0:r1], dk[:, r0:r1], dv[:, r0:r1]))
        if lens[b] >= 2048:
            for name, a, ref in (("o", got[0], do_[0]), ("lse", got[1], dl[0]), ("dq", got[2][0], dq_[0])):
                assert np.array_equal(a, ref), f"sequence {b} {name} differs from the dense call"
            # The dense call's dK/dV kernel splits each workgroup's query tiles between two
            # wave groups when its grid (128-key tiles x KV heads) has at most 768
            # workgroups, three per CU, at D = 128; dK and dV are then the sum of two fp32 partial sums
            # instead of one running sum.  The order changes the fp32 rounding (relative to
            # the terms, which can be far larger than a cancelling result) and so, here and
            # there, the bf16 value: the two must agree to half a bf16 step of the tensor's
            # largest value and to 1e-3 in rel-L2.  Otherwise the kernels match bit for bit.
            split = -(-lens[b] // 128) * Hkv <= 3 * 256
            for name, a, ref in (("dk", got[2][1], dk_[0]), ("dv", got[2][2], dv_[0])):
                if not split:
                    assert np.array_equal(a, ref), f"sequence {b} {name} differs from the dense call"
                else:
                    a64, r64 = a.astype(np.float64), ref.astype(np.float64)
                    worst = float(np.abs(a64 - r64).max())
                    assert worst <= 2.0 ** -8 * float(np.abs(r64).max()), f"sequence {b} {name}: max diff {worst:.3g}"
                    e = rel_l2(a64, r64)
                    assert e <= 1e-3, f"sequence {b} {name}: rel-L2 {e:.3g} against the dense call"
        else:
            # the dense call takes other kernels here, so both are held to the oracle
            ref = oracle.sdpa_backward(sub["q"], sub["k"], sub["v"], sub["do"], scale, True)
            compare(got, {n: ref[n][0] for n in ("o", "lse", "dq", "dk", "dv")}, dtype,
                    f"packed sequence {b} against the oracle")
            compare((do_[0], dl[0], (dq_[0], dk_[0], dv_[0])), {n: ref[n][0] for n in ("o", "lse", "dq", "dk", "dv")},
                    dtype, f"dense call of sequence {b} against the oracle")
    rng = np.random.default_rng(5)
    dq_got, dq_ref = [], []
    for b in (0, 2, 4, 9):
        r0, n = int(cu[b]), lens[b]
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
        for h in (0, 13, 31):
            sub = {x: inp[x][None, :, r0:r0 + n] for x in ("q", "k", "v", "do")}
            O, L = oracle.sdpa_forward_rows(sub["q"], sub["k"], sub["v"], scale, True, 0, h, rows)
            check_o(o[h, r0 + rows], O, dtype, f"seq {b} head {h}")
            check_lse(lse[h, r0 + rows], L, dtype, f"seq {b} head {h}")
            dq_ref.append(oracle.sdpa_dq_rows(sub["q"], sub["k"], sub["v"], sub["do"], scale, True, 0, h, rows))
            dq_got.append(dq[h, r0 + rows])
    e = rel_l2(np.concatenate(dq_got), np.concatenate(dq_ref))
    assert e <= TOL[dtype]["grad"], f"sampled dQ rows rel-L2 {e:.3e}"


def test_equal_lengths_ex_matches_plain_bitwise():
    """fa_fwd_ex / fa_bwd_ex with Sq = Skv and no window is the plain problem."""
    B, Hq, Hkv, S, D = 2, 4, 2, 333, 128
    inp = make_inputs(B, Hq, Hkv, S, D, "bf16", seed=11)
    q, k, v, do = (dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(D)
    say("case ex == plain")
    o1, l1 = fa.forward(q, k, v, scale=scale)
    g1 = fa.backward(q, k, v, o1, l1, do, scale=scale)
    s = torch.cuda.current_stream().cuda_stream
    p = fa.params(B, Hq, Hkv, S, S, D, scale, True, None, fa.FA_BF16)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    assert fa.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), p, s) == fa.FA_OK
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    ws = torch.empty(fa.fa_bwd_ex_workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    st = fa.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), do.data_ptr(),
                      *(t.data_ptr() for t in g2), p, ws.data_ptr(), ws.numel(), s)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


WIDE = [(False, None, 2048, 2048, 128), (True, 300, 2048, 2048, 128), (False, 700, 2048, 2048, 128),
        (True, None, 1999, 1999, 128), (False, None, 1999, 1999, 128), (True, None, 1800, 2113, 128),
        (False, None, 2001, 1937, 128), (True, 450, 2040, 2040, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal,window,S,Skv,D", WIDE)
def test_wide_grid_masks(causal, window, S, Skv, D, dtype):
    """A grid large enough for the 8-wave workgroups of the forward and dQ kernels
    (B=8, 32/8 heads: ceil(Sq/256) * 8 * 32 = 2048 eight-wave query blocks, which
    dispatches the 8-wave forward at D = 128 from 256 and at D = 64 from 2048, and
    the 8-wave dQ from 2048), in bf16 and fp16, with the causal, non-causal and
    windowed masks, key counts that end inside a 128-key load stage and keys longer
    or shorter than the queries: sampled rows of every head against the oracle, and
    one whole KV group's gradients."""
    B, Hq, Hkv = 8, 32, 8
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=4200 + (window or 0) + S + Skv + D, q_std=2.0, Skv=Skv)
    what = f"wide grid {dtype} causal={causal} window={window} Sq={S} Skv={Skv} D={D}"
    say("case", what)
    o, lse, (dq, dk, dv) = run_dense(inp, dtype, scale, causal, window)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, S - 1], rng.integers(0, S, 5)]))
    for b in (0, 7):
        for h in range(0, Hq, 5):
            Or, Lr = oracle.sdpa_forward_rows(inp["q"], inp["k"], inp["v"], scale, causal, b, h, rows, window=window)
            check_o(o[b, h, rows], Or, dtype, f"{what} b={b} h={h}")
            check_lse(lse[b, h, rows], Lr, dtype, f"{what} b={b} h={h}")
    g = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, groups=[(3, 5)], window=window)
    heads = list(range(5 * 4, 6 * 4))
    check_o(o[3, heads], g["o"][3, heads], dtype, what + " group")
    check_grads((dq[3, heads], dk[3, 5], dv[3, 5]), (g["dq"][3, heads], g["dk"][3, 5], g["dv"][3, 5]), dtype, what)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal,window,S", [(True, None, 2048), (True, None, 1999), (False, 600, 2048)])
def test_mid_grid_dkdv(causal, window, S, dtype):
    """B = 4, 32/8 heads, D = 128: ceil(S/128) * 4 * 8 = 512 four-wave key blocks, two
    per CU, which dispatches the dK/dV kernel's two-group form beyond one workgroup per
    CU (and, with 8-wave query blocks from 256, the 8-wave forward).  One whole KV
    group's O and gradients against the oracle, and sampled rows of the gradients of
    every other KV head (and the last)."""
    B, Hq, Hkv, D = 4, 32, 8, 128
    scale = 1.0 / math.sqrt(D)
    inp = make_inputs(B, Hq, Hkv, S, D, dtype, seed=4700 + S + (window or 0), q_std=2.0)
    what = f"mid-grid dK/dV {dtype} causal={causal} window={window} S={S}"
    say("case", what)
    o, lse, (dq, dk, dv) = run_dense(inp, dtype, scale, causal, window)
    b, g = 2, 6
    ref = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, groups=[(b, g)], window=window)
    heads = list(range(g * 4, (g + 1) * 4))
    check_o(o[b, heads], ref["o"][b, heads], dtype, what + " group")
    check_grads((dq[b, heads], dk[b, g], dv[b, g]), (ref["dq"][b, heads], ref["dk"][b, g], ref["dv"][b, g]),
                dtype, what)
    rows = np.array([0, 1, 31, 32, 255, 256, S // 2, S - 2, S - 1])
    for bb in (0, 3):
        for kh in (0, 2, 4, 7):
            r = oracle.sdpa_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, groups=[(bb, kh)],
                                     window=window)
            check_grads((dq[bb, kh * 4:(kh + 1) * 4, rows], dk[bb, kh, rows], dv[bb, kh, rows]),
                        (r["dq"][bb, kh * 4:(kh + 1) * 4, rows], r["dk"][bb, kh, rows], r["dv"][bb, kh, rows]),
                        dtype, f"{what} b={bb} kv={kh}")
