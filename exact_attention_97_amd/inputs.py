"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to bfloat16; it holds
none of attention's arithmetic.  Both the parity tests (GPU path against the
CPU oracle) and the benchmark draw their inputs from here, so the two sides
always see identical bf16 values.

Recipe (the pages print no benchmark shapes; these workloads stand in):
* float32 draws from ``torch.Generator().manual_seed(seed)`` in the order
  Q, K, V, dO, then the outlier masks of Q and of K;
* values are ``randn * std``;
* outliers: an independent Bernoulli(frac) mask per entry of Q and of K
  multiplies the float32 value by ``outlier_scale`` before rounding;
* the float32 values are rounded to bfloat16 (round to nearest even).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: tuple  # which causal settings the workload covers
    seed: int
    std: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 20.0
    passes: str = "fwd+bwd"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The workloads, smallest first.  Sizes are [B, H, S, D].
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, (False,), seed=0),
    "fwd2k": Workload("fwd2k", 8, 16, 2048, 128, (False, True), seed=1, passes="fwd"),
    "long8k": Workload("long8k", 2, 16, 8192, 128, (False, True), seed=2,
                       outlier_frac=0.01, outlier_scale=20.0, passes="fwd"),
    "bwd4k": Workload("bwd4k", 4, 16, 4096, 128, (False, True), seed=3),
    "ctx32k": Workload("ctx32k", 1, 32, 32768, 128, (True,), seed=4, std=0.5),
    "d64": Workload("d64", 2, 16, 8192, 64, (False, True), seed=5, std=0.5),
    "d256": Workload("d256", 2, 16, 8192, 256, (False, True), seed=6, std=0.5),
    "bwd8k": Workload("bwd8k", 2, 16, 8192, 128, (False, True), seed=7),
}


def make_qkvdo(B, H, S, D, seed, std=1.0, outlier_frac=0.0, outlier_scale=20.0):
    """Draw Q, K, V, dO as CPU bfloat16 tensors of shape [B, H, S, D]."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, S, D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        q.mul_(std)
        k.mul_(std)
        v.mul_(std)
        do.mul_(std)
    if outlier_frac > 0.0:
        mq = torch.rand(shape, generator=g) < outlier_frac
        mk = torch.rand(shape, generator=g) < outlier_frac
        q[mq] *= outlier_scale
        k[mk] *= outlier_scale
    return (q.to(torch.bfloat16), k.to(torch.bfloat16),
            v.to(torch.bfloat16), do.to(torch.bfloat16))


def make_workload(w: Workload):
    """Inputs of a named workload (CPU bf16 tensors)."""
    return make_qkvdo(w.B, w.H, w.S, w.D, w.seed, w.std, w.outlier_frac, w.outlier_scale)


def make_qkv_rect(B, H, Sq, Sk, D, seed, std=1.0):
    """Draw Q [B, H, Sq, D] and K, V [B, H, Sk, D] (in that order) as CPU bfloat16
    tensors, for queries and keys of different lengths (split-KV forward)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Sq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Sk, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Sk, D), generator=g, dtype=torch.float32)
    if std != 1.0:
        q.mul_(std)
        k.mul_(std)
        v.mul_(std)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@dataclass(frozen=True)
class RectWorkload:
    """A forward workload with Sq queries over Sk keys (split-KV forward)."""

    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed: int
    std: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# Long key sequences with few queries: one decoding step per sequence, and a
# 512-query chunk of prefill continuing a 32k context (causal, the queries
# being the last 512 positions).
SPLITKV_WORKLOADS = {
    "decode32k": RectWorkload("decode32k", B=4, H=32, Sq=1, Sk=32768, D=128, causal=True, seed=8, std=0.5),
    "prefill32k": RectWorkload("prefill32k", B=1, H=32, Sq=512, Sk=32768, D=128, causal=True, seed=9, std=0.5),
}


def hadamard_signs(D, seed):
    """The random signs of the FP8 path's transform: float32 [D] of +1 / -1 (CPU),
    from an independent seeded generator (one uniform draw per element)."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand((D,), generator=g, dtype=torch.float64)
    return torch.where(u < 0.5, -1.0, 1.0).to(torch.float32)
