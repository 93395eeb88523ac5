"""Seeded synthetic workloads.

This module only draws random inputs and names the workload shapes; it holds
none of the method's arithmetic (no packing, decoding or matmul).  Both the
oracle side and the HIP side take their inputs from here.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload, in this
order):
  1. W f32 [n,k] = sigma * standard_normal.
  2. Only for the outlier workloads: exactly floor(0.01*n*k) distinct flat
     indices from ``rng.choice(n*k, size, replace=False)``, multiplied by 50.
  3. X f32 [m,k] = standard_normal, then rounded to bf16 (round to nearest
     even, via torch's dtype conversion) where the workload's activation is
     bf16.

The shapes follow the decode GEMV / prefill GEMM shapes of the pages (decode
at n=k=4096, a 14336x4096 MLP projection with outliers, prefill at
m=2048, n=k=4096, and an 11008x4096 projection at m=512); no public dataset
is involved and no trained weights are needed.

The expert-routed workload draws the stacked weights (step 1), then the
routing (draw_expert_ids), then X (step 3) from its own stream; it stands in
for a prefill-scale MoE layer's routed tokens.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    m: int
    n: int
    k: int
    sigma: float
    outliers: bool
    act: str  # "f32" or "bf16": dtype of X and of the output
    seed: int
    op: str  # "qgemv" (m == 1) or "qgemm"
    tol: float  # |gpu - ref| <= tol * sum|x*w|

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("mxfp4_m8_n16_k512", "mxfp4", 8, 16, 512, 1.0, False, "f32", 1000, "qgemm", 1e-5),
        Workload("nvfp4_qgemv_4096", "nvfp4", 1, 4096, 4096, 0.02, False, "bf16", 1001, "qgemv", 2e-3),
        Workload("mxfp8_e4m3_qgemv_14336", "mxfp8_e4m3", 1, 14336, 4096, 0.02, True, "bf16", 1002, "qgemv", 2e-3),
        Workload("mxfp8_e5m2_qgemv_14336", "mxfp8_e5m2", 1, 14336, 4096, 0.02, True, "bf16", 1002, "qgemv", 2e-3),
        Workload("mxfp4_qgemm_2048", "mxfp4", 2048, 4096, 4096, 0.02, False, "bf16", 1003, "qgemm", 2e-3),
        Workload("int4_affine_qgemm_512", "int4_affine", 512, 11008, 4096, 0.02, False, "bf16", 1004, "qgemm", 2e-3),
        Workload("int8_sym_qgemm_512", "int8_sym", 512, 11008, 4096, 0.02, False, "bf16", 1004, "qgemm", 2e-3),
    ]
}


@dataclass(frozen=True)
class MoeWorkload:
    """A prefill-scale expert-routed matmul: `tokens` tokens, each routed to
    `topk` distinct experts of `experts`, every expert an [n, k] weight packed
    in one [experts*n, k] stack; m = tokens*topk routed rows (token-major)."""
    name: str
    fmt: str
    tokens: int
    topk: int
    experts: int
    n: int
    k: int
    sigma: float
    seed: int
    tol: float

    @property
    def m(self) -> int:
        return self.tokens * self.topk

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


MOE_WORKLOADS = {
    w.name: w
    for w in [
        # 1024 tokens, top-2 of 8 experts of 4096 x 4096 (mxfp4): 2048 routed
        # rows, the flops of the dense m=2048 prefill over 8x its weight bytes
        MoeWorkload("mxfp4_moe_prefill_8x4096", "mxfp4", 1024, 2, 8, 4096, 4096, 0.02, 1006, 2e-3),
    ]
}


def draw_expert_ids(tokens: int, topk: int, experts: int, rng) -> np.ndarray:
    """Routed expert ids, int32 [tokens*topk] (token-major): per token, the
    topk largest of experts standard-normal scores plus a per-expert offset
    (drawn once, 0.5 * standard normal) that makes the expert loads uneven."""
    bias = np.float32(0.5) * rng.standard_normal(experts, dtype=np.float32)
    scores = rng.standard_normal((tokens, experts), dtype=np.float32) + bias
    top = np.argsort(-scores, axis=1, kind="stable")[:, :topk]
    return np.ascontiguousarray(top.reshape(-1), dtype=np.int32)


def generate_moe(w: MoeWorkload | str, tokens: int | None = None):
    """(W stack f32 [experts*n, k], X f32 [tokens*topk, k] bf16 values, ids)
    for an expert-routed workload: weights, then ids, then activations from
    one seeded stream."""
    if isinstance(w, str):
        w = MOE_WORKLOADS[w]
    t = w.tokens if tokens is None else tokens
    rng = np.random.default_rng(w.seed)
    W = draw_weights(w.experts * w.n, w.k, w.sigma, False, rng)
    ids = draw_expert_ids(t, w.topk, w.experts, rng)
    X = draw_activations(t * w.topk, w.k, "bf16", rng)
    return W, X, ids


def draw_weights(n: int, k: int, sigma: float, outliers: bool, rng) -> np.ndarray:
    w = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    if outliers:
        cnt = (n * k) // 100
        idx = rng.choice(n * k, size=cnt, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(50.0)
    return w


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (RNE) with torch; return the f32 values of the result."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def draw_activations(m: int, k: int, act: str, rng) -> np.ndarray:
    x = rng.standard_normal((m, k), dtype=np.float32)
    if act == "bf16":
        x = to_bf16_values(x)
    return x


def generate(w: Workload | str, m: int | None = None, n: int | None = None, k: int | None = None):
    """Return (W f32 [n,k], X f32 [m,k]) for a workload; m/n/k may be
    overridden (same recipe, smaller shape) for oracle-sized parity cases."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    m = w.m if m is None else m
    n = w.n if n is None else n
    k = w.k if k is None else k
    rng = np.random.default_rng(w.seed)
    W = draw_weights(n, k, w.sigma, w.outliers, rng)
    X = draw_activations(m, k, w.act, rng)
    return W, X


def random_weights(n: int, k: int, seed: int, sigma: float = 1.0, outliers: bool = False) -> np.ndarray:
    return draw_weights(n, k, sigma, outliers, np.random.default_rng(seed))


def random_activations(m: int, k: int, seed: int, act: str = "bf16") -> np.ndarray:
    return draw_activations(m, k, act, np.random.default_rng(seed))
