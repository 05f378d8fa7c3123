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
    """N is the key count; N_q (default N) the query rows.  N_q < N is a
    prefill chunk against a KV cache, N_q = 1 a decode step."""
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    D: int
    causal: bool
    seed: int
    N_q: int | None = None

    @property
    def Nq(self) -> int:
        return self.N if self.N_q is None else self.N_q

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_shape(self):
        return (self.B, self.H_q, self.Nq, self.D)

    def kv_shape(self):
        return (self.B, self.H_kv, self.N, self.D)

    def flops(self) -> float:
        """Attention FLOPs: two contractions of 2*D per visible (query, key) pair
        per head.  Causal counts N_q*N - N_q^2/2 pairs (N^2/2 when square)."""
        pairs = float(self.Nq) * self.N
        if self.causal:
            pairs -= float(self.Nq) * self.Nq / 2
        return 4.0 * self.B * self.H_q * pairs * self.D

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once (bf16) plus O (bf16) and LSE (fp32) written once."""
        qo = self.B * self.H_q * self.Nq * self.D * 2
        kv = self.B * self.H_kv * self.N * self.D * 2
        lse = self.B * self.H_q * self.Nq * 4
        return 2 * qo + 2 * kv + lse

    def bwd_algorithmic_bytes(self) -> int:
        """The backward's Q, K, V, O, dO (bf16) and LSE (fp32) read once and
        dQ, dK, dV (bf16) written once."""
        qo = self.B * self.H_q * self.Nq * self.D * 2
        kv = self.B * self.H_kv * self.N * self.D * 2
        lse = self.B * self.H_q * self.Nq * 4
        return 4 * qo + 4 * kv + lse


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
    # one decode step (one query row) against a KV cache: the softmax-decode
    # shape B=1, H=32, D=128 of the page "Attention Kernel 实现与正确性验证",
    # section 3.5.1, at its three context lengths, plus a GQA-4 variant
    Workload("decode_mha_n4096", 1, 32, 32, 4096, 128, True, 601, N_q=1),
    Workload("decode_mha_n16384", 1, 32, 32, 16384, 128, True, 602, N_q=1),
    Workload("decode_mha_n65536", 1, 32, 32, 65536, 128, True, 603, N_q=1),
    Workload("decode_gqa4_n65536", 1, 32, 8, 65536, 128, True, 604, N_q=1),
    # a 512-row prefill chunk appended to an 8192-key cache (bottom-right causal)
    Workload("chunk_gqa4_q512_n8192", 1, 32, 8, 8192, 128, True, 605, N_q=512),
]
WORKLOADS = {w.name: w for w in _W}

# The long-context causal GQA-4 workload at N=32768 is the headline measurement.
HEADLINE = "gqa4_n32768_causal"


def make_inputs(B: int, H_q: int, H_kv: int, N: int, D: int, seed: int,
                dist: str = "normal", N_kv: int | None = None):
    """Draw bf16 Q [B,H_q,N,D], K and V [B,H_kv,N_kv,D] (N_kv defaults to N) on the CPU.

    dist="normal": i.i.d. N(0,1) float32 rounded to bf16 (the workloads' recipe).
    dist="uniform": i.i.d. U(-1,1), used by a few edge-case tests.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    nk = N if N_kv is None else N_kv
    shapes = [(B, H_q, N, D), (B, H_kv, nk, D), (B, H_kv, nk, D)]
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
    return make_inputs(w.B, w.H_q, w.H_kv, w.Nq, w.D, w.seed, N_kv=w.N)


def to_float64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 (or fp32) CPU tensor to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


# ---------------------------------------------------------------- MLA decode
@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    """Absorbed MLA decode, DeepSeek-V3 shapes of page "Attention Kernel 实现与
    正确性验证", section 2.3: H=128 heads, latent d_c=512, rotary d_R=64,
    d_nope = d_v = 128, S query tokens against a T-token latent cache."""
    name: str
    B: int
    S: int
    T: int
    seed: int
    H: int = 128
    d_c: int = 512
    d_r: int = 64
    d_nope: int = 128
    d_v: int = 128
    causal: bool = True

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_nope + self.d_r)

    def core_flops(self) -> float:
        """Latent attention: 2*(d_c + d_r) + 2*d_c per visible (token, head, key)."""
        pairs = float(self.S) * self.T - (float(self.S) * (self.S - 1) / 2 if self.causal else 0.0)
        return self.B * self.H * pairs * 2.0 * (2 * self.d_c + self.d_r)

    def core_bytes(self) -> int:
        """Latent cache read once, absorbed queries read, latent outputs and LSE written."""
        kv = self.B * self.T * (self.d_c + self.d_r) * 2
        q = self.B * self.H * self.S * (self.d_c + self.d_r) * 2
        o = self.B * self.H * self.S * (self.d_c * 2 + 4)
        return kv + q + o


MLA_WORKLOADS = {w.name: w for w in [
    MlaWorkload("mla_decode_t4096", 1, 1, 4096, 701),
    MlaWorkload("mla_decode_t16384", 1, 1, 16384, 702),
    MlaWorkload("mla_decode_b8_t4096", 8, 1, 4096, 703),
    MlaWorkload("mla_decode_b32_t4096", 32, 1, 4096, 704),
]}


def make_mla_inputs(B: int, H: int, S: int, T: int, seed: int, d_c: int = 512, d_r: int = 64,
                    d_nope: int = 128, d_v: int = 128):
    """Draw bf16 c_kv [B,T,d_c], k_pe [B,T,d_r], q_nope [B,H,S,d_nope],
    q_pe [B,H,S,d_r], W_uk [H,d_nope,d_c], W_uv [H,d_v,d_c] on the CPU, in that
    order from one seeded generator: i.i.d. N(0,1), the two projections scaled
    by 1/sqrt(d_c) so that reconstructed keys and values are about N(0,1)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shapes = [(B, T, d_c), (B, T, d_r), (B, H, S, d_nope), (B, H, S, d_r), (H, d_nope, d_c),
              (H, d_v, d_c)]
    out = []
    for i, s in enumerate(shapes):
        t = torch.randn(s, generator=g, dtype=torch.float32)
        if i >= 4:
            t = t / math.sqrt(d_c)
        out.append(t.to(torch.bfloat16))
    return tuple(out)
