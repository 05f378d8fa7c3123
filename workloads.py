"""Seeded synthetic inputs for the attention forward: shapes, seeds, generator.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
benchmark and the smoke check.  It holds no attention arithmetic: it only names
the workloads and draws their Q, K, V tensors.

Workload shapes follow the numerical-check shapes of the page "Attention Kernel
实现与正确性验证" (section 1.3: GQA-4, GQA-8, MHA, MQA at D=128, written there as
[B-Hq-Hkv-N-D]) and the sequence-length sweep of its section 1.4 (N up to 32768).
Values are i.i.d. standard normal in float32, rounded to bfloat16
(round-to-nearest-even), drawn in the order Q, K, V from one CPU generator
seeded per workload.  No dataset is involved: the pages' shapes are
model-shaped (LLaMA-3-like head counts), not drawn from a benchmark suite.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    D: int
    causal: bool
    seed: int

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_shape(self):
        return (self.B, self.H_q, self.N, self.D)

    def kv_shape(self):
        return (self.B, self.H_kv, self.N, self.D)

    def flops(self) -> float:
        """Attention FLOPs: two contractions of 2*N*N*D each per (b, h_q), halved when causal."""
        f = 4.0 * self.B * self.H_q * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once (bf16) plus O (bf16) and LSE (fp32) written once."""
        qo = self.B * self.H_q * self.N * self.D * 2
        kv = self.B * self.H_kv * self.N * self.D * 2
        lse = self.B * self.H_q * self.N * 4
        return 2 * qo + 2 * kv + lse


_W = [
    Workload("tiny_mha_n256_d64", 1, 4, 4, 256, 64, False, 101),
    Workload("gqa4_b2_n1024", 2, 32, 8, 1024, 128, True, 201),
    Workload("mha_n512", 1, 32, 32, 512, 128, True, 301),
    Workload("mqa_n512", 1, 16, 1, 512, 128, True, 302),
    Workload("gqa8_n4096_causal", 1, 64, 8, 4096, 128, True, 401),
    Workload("gqa8_n4096_full", 1, 64, 8, 4096, 128, False, 401),
    Workload("gqa4_n8192_causal", 1, 32, 8, 8192, 128, True, 508),
    Workload("gqa4_n16384_causal", 1, 32, 8, 16384, 128, True, 516),
    Workload("gqa4_n32768_causal", 1, 32, 8, 32768, 128, True, 532),
]
WORKLOADS = {w.name: w for w in _W}

# The long-context causal GQA-4 workload at N=32768 is the headline measurement.
HEADLINE = "gqa4_n32768_causal"


def make_inputs(B: int, H_q: int, H_kv: int, N: int, D: int, seed: int,
                dist: str = "normal"):
    """Draw bf16 Q [B,H_q,N,D], K and V [B,H_kv,N,D] on the CPU.

    dist="normal": i.i.d. N(0,1) float32 rounded to bf16 (the workloads' recipe).
    dist="uniform": i.i.d. U(-1,1), used by a few edge-case tests.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shapes = [(B, H_q, N, D), (B, H_kv, N, D), (B, H_kv, N, D)]
    out = []
    for s in shapes:
        if dist == "normal":
            t = torch.randn(s, generator=g, dtype=torch.float32)
        elif dist == "uniform":
            t = torch.rand(s, generator=g, dtype=torch.float32) * 2 - 1
        else:
            raise ValueError(dist)
        out.append(t.to(torch.bfloat16))
    return tuple(out)


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H_q, w.H_kv, w.N, w.D, w.seed)


def to_float64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 (or fp32) CPU tensor to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
