"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no attention arithmetic: it only names the workload shapes and draws
and rounds random tensors.  Both the HIP path and the oracle consume the exact
same rounded values, so any difference between them comes from the method,
never from the inputs.

Shapes follow the pages' workloads: GPT-2-small heads (12 x 64) and Qwen3-style
GQA (32 query heads over 8 KV heads, head dim 128) from "Phase 14: Flash
Attention 2 for SM120" (kernel configuration and GQA sections), the
[1, 8, 4096, 64] fp16 causal tensor of "FlashAttention 与 SDPA Backend"
(memory and IO section) and of the udemi.tech "Flash Attention" usage snippet.

Recipe (per workload): ``rng = numpy.random.default_rng(seed)``; draw q, k, v
and then dO (when the workload has a backward pass), each as a float32
``standard_normal`` of its full shape; q is multiplied by ``q_std``; each tensor
is then rounded to the workload dtype with round-to-nearest-even.  The rounded
values are returned as float32 arrays, which hold bf16 / fp16 values exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    seed: int
    q_std: float = 1.0
    backward: bool = True
    causal: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def causal_pairs(self) -> int:
        """(query, key) pairs the causal method must visit, over all heads."""
        per_head = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return self.B * self.Hq * per_head

    def fwd_flops(self) -> float:
        # QK^T and PV: 2 * D flops each per visited pair.
        return 4.0 * self.D * self.causal_pairs()

    def bwd_flops(self) -> float:
        # five products per visited pair (S recompute, dP, dV, dK, dQ).
        return 10.0 * self.D * self.causal_pairs()


# The five workloads, named by what they are.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("causal_f32_b1_h2_s128_d64", "f32", 1, 2, 2, 128, 64, seed=0),
        Workload("gpt2s_causal_bf16_b8_h12_s1024_d64", "bf16", 8, 12, 12, 1024, 64, seed=1),
        Workload("qwen3_gqa_causal_bf16_b4_h32kv8_s2048_d128", "bf16", 4, 32, 8, 2048, 128,
                 seed=2, backward=False),
        Workload("causal_f16_b1_h8_s4096_d64", "f16", 1, 8, 8, 4096, 64, seed=3),
        Workload("longctx_gqa_causal_bf16_b1_h32kv8_s16384_d128", "bf16", 1, 32, 8, 16384, 128,
                 seed=4, q_std=3.0),
    )
}
SMALL = "causal_f32_b1_h2_s128_d64"


@dataclass(frozen=True)
class DecodeWorkload:
    """Decoding against a KV cache: Sq new query rows per sequence, Skv cached keys,
    the causal diagonal aligned to the last key (bottom-right)."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def pairs(self) -> int:
        # query row i of Sq sees keys 0 .. Skv - Sq + i
        per_head = sum(max(0, min(self.Skv, self.Skv - self.Sq + i + 1)) for i in range(self.Sq))
        return self.B * self.Hq * per_head

    def flops(self) -> float:
        return 4.0 * self.D * self.pairs()

    def min_bytes(self) -> int:
        """Bytes a decode step must move: K, V once per KV head; Q, O; fp32 L."""
        e = 4 if self.dtype == "f32" else 2
        kv = 2 * self.B * self.Hkv * self.Skv * self.D * e
        qo = 2 * self.B * self.Hq * self.Sq * self.D * e
        return kv + qo + 4 * self.B * self.Hq * self.Sq


# One decode step of the Qwen3-style GQA shape (32 query heads over 8 KV heads,
# head dim 128) for a batch of 16 sequences with 8192 cached keys each.
DECODE = DecodeWorkload("decode_qwen3_gqa_bf16_b16_h32kv8_sq1_skv8192_d128", "bf16", 16, 32, 8, 1, 8192, 128,
                        seed=5)
LONG_CONTEXT = "longctx_gqa_causal_bf16_b1_h32kv8_s16384_d128"


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(B, Hq, Hkv, S, D, dtype, seed, q_std=1.0, backward=True, Skv=None):
    """Draw q, k, v (and dO) per the recipe above.  Returns a dict of float32 arrays.

    q and dO are [B,Hq,S,D]; k and v are [B,Hkv,Skv,D] (Skv defaults to S)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    Skv = S if Skv is None else Skv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    if q_std != 1.0:
        q *= np.float32(q_std)
    k = rng.standard_normal((B, Hkv, Skv, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D), dtype=np.float32)
    out = {"q": round_to(q, dtype), "k": round_to(k, dtype), "v": round_to(v, dtype)}
    if backward:
        out["do"] = round_to(rng.standard_normal((B, Hq, S, D), dtype=np.float32), dtype)
    return out


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.seed, w.q_std, w.backward)


def make_varlen_inputs(seqlens_q, seqlens_k, Hq, Hkv, D, dtype, seed, q_std=1.0):
    """A packed batch: sequence b has seqlens_q[b] query rows and seqlens_k[b] key rows.

    Returns float32 arrays q, dO [Hq,Tq,D], k, v [Hkv,Tk,D] (rows of all
    sequences back to back within each head) and the int32 offset vectors
    cu_q, cu_k of length B + 1 (cu[b] is the first row of sequence b)."""
    if len(seqlens_q) != len(seqlens_k):
        raise ValueError("one key length per query length")
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, Tq, D), dtype=np.float32) * np.float32(q_std)
    k = rng.standard_normal((Hkv, Tk, D), dtype=np.float32)
    v = rng.standard_normal((Hkv, Tk, D), dtype=np.float32)
    do = rng.standard_normal((Hq, Tq, D), dtype=np.float32)
    return {"q": round_to(q, dtype), "k": round_to(k, dtype), "v": round_to(v, dtype),
            "do": round_to(do, dtype), "cu_q": cu_q, "cu_k": cu_k}


def decode_inputs(w: DecodeWorkload):
    return make_inputs(w.B, w.Hq, w.Hkv, w.Sq, w.D, w.dtype, w.seed, backward=False, Skv=w.Skv)
