"""Seeded synthetic inputs for the verify step.

This module only draws random numbers and rounds them to the storage formats
the workloads name (bf16 activations, fp32 weights and logits).  It holds none
of the method's arithmetic: no quantisation, no GEMM, no warp, no acceptance.
It is the single module shared by the product tests/benchmark and the CPU
oracle, so both sides see bit-identical inputs.

Workloads (shapes and distributions):
  * LM-head verify: hidden d=1024 bf16 rows ~N(0,1), M=4 rows (3 drafts + bonus),
    vocab V=8192, weights ~N(0,0.02); draft logits ~N(0,2) fp32 whose softmax is
    the draft distribution q; temperature 0.6, top_p 0.95.  A V=16 variant of the
    same recipe drives the tiny-vocabulary distribution trials.
  * Dense 27B-class decoder layer linears: d_model 5120, 40 query heads and 8
    KV heads of dim 128, SwiGLU width 17408; activations bf16 ~N(0,1).
  * Large-vocab verify: d=5120, V=151936, draft logits ~N(0,3).
  * MoE verify: 128 experts, top-8, d_model 2048, expert FFN width 768.
"""
from __future__ import annotations

import numpy as np

# numpy PCG64 seeds per workload and the Philox key seeds of the verify step.
SEED_BASE = 20261200
PHILOX_SEED_BASE = 0x5EED0000

LM_SMALL = dict(d=1024, V=8192, M=4, w_std=0.02, draft_std=2.0, T=0.6, top_p=0.95)
LM_TINY = dict(d=1024, V=16, M=4, w_std=0.02, draft_std=2.0, T=0.6, top_p=0.95)
LAYER27B = dict(d_model=5120, n_q=40, n_kv=8, head=128, ffn=17408, w_std=0.02)
LM_LARGE = dict(d=5120, V=151936, M=4, w_std=0.02, draft_std=3.0)
MOE = dict(n_exp=128, topk=8, d_model=2048, ffn=768, V=151936, w_std=0.02, draft_std=3.0)

# name -> (N, K) of the dense layer's linears, fused forms included
LAYER27B_LINEARS = {
    "q": (5120, 5120), "k": (1024, 5120), "v": (1024, 5120), "o": (5120, 5120),
    "gate": (17408, 5120), "up": (17408, 5120), "down": (5120, 17408),
    "qkv": (7168, 5120), "gate_up": (34816, 5120),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round binary32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Used only to put synthetic activations into their storage format."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def softmax_f32(logits: np.ndarray) -> np.ndarray:
    """Draft distribution q from draft logits: computed in fp64, stored fp32.
    This is input preparation (the drafter's output), not the verify method."""
    l = np.asarray(logits, dtype=np.float64)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def sample_drafts(g: np.random.Generator, q: np.ndarray, B: int) -> np.ndarray:
    """Drafts x_i ~ q_i for B independent problems: int32 [B][D].
    Stands in for the multi-token-prediction head's own draws."""
    q = np.asarray(q, dtype=np.float64)
    D, V = q.shape
    out = np.empty((B, D), dtype=np.int32)
    for i in range(D):
        c = np.cumsum(q[i])
        u = g.random(B) * c[-1]
        out[:, i] = np.minimum(np.searchsorted(c, u, side="right"), V - 1)
    return out


def lm_verify_problem(cfg: dict, seed: int, B: int = 1):
    """Hidden rows, fp32 LM-head weights, draft logits, q and drafts."""
    g = rng(seed)
    d, V, M = cfg["d"], cfg["V"], cfg["M"]
    D = M - 1
    w = normal_f32(g, (V, d), cfg["w_std"])
    x = f32_to_bf16_bits(normal_f32(g, (M, d), 1.0))
    draft_logits = normal_f32(g, (D, V), cfg["draft_std"])
    q = softmax_f32(draft_logits)
    drafts = sample_drafts(g, q, B)
    return dict(w=w, x=x, draft_logits=draft_logits, q=q, drafts=drafts)


def synthetic_logits(seed: int, rows: int, V: int, std: float) -> np.ndarray:
    """fp32 logits ~N(0, std) (stand-in for LM-head outputs in stage-isolated tests)."""
    return normal_f32(rng(seed), (rows, V), std)


def q_and_drafts(seed: int, D: int, V: int, std: float, B: int = 1):
    g = rng(seed)
    ql = normal_f32(g, (D, V), std)
    q = softmax_f32(ql)
    return q, sample_drafts(g, q, B)


def linear_weights(seed: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    return normal_f32(rng(seed), (N, K), std)


def activations_bf16(seed: int, M: int, K: int, std: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(rng(seed), (M, K), std))
