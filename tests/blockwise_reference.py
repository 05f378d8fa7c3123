"""Blockwise online-softmax attention in float64 (test code, used only as a pin).

An independent second route to the attention result: the running-statistics
recurrence of the flash-attention forward, taken over query tiles of `tile_m`
rows and key tiles of `tile_n` keys (page "Attention Kernel 实现与正确性验证",
section 1.2; page "Flash Attention 与 Kernel 优化", section "running softmax
状态"; page "Triton Cuda Attention", section "在线 Softmax 核心算法").  Per key
tile, for each row:

    m_new = max(m, rowmax(s))
    alpha = exp(m - m_new)
    p     = exp(s - m_new)
    l     = alpha * l + rowsum(p)
    acc   = alpha * acc + p @ V_tile
    m     = m_new

then O = acc / l and LSE = m + log(l).  The pages start l at 0 in two places and
at 1.0 in one; both are accepted (`l_init`), since the first update multiplies
l by alpha = exp(-inf) = 0.  The causal loop stops at the query tile's last row.
"""
from __future__ import annotations

import numpy as np


def blockwise_attention(q, k, v, *, is_causal, sm_scale, tile_m=16, tile_n=16,
                        l_init=0.0):
    B, H_q, N, D = q.shape
    H_kv = k.shape[1]
    O = np.zeros((B, H_q, N, D))
    L = np.zeros((B, H_q, N))
    for b in range(B):
        for h in range(H_q):
            g = (h * H_kv) // H_q
            for m0 in range(0, N, tile_m):
                rows = np.arange(m0, min(m0 + tile_m, N))
                qt = q[b, h, rows]
                m = np.full(rows.size, -np.inf)
                l = np.full(rows.size, float(l_init))
                acc = np.zeros((rows.size, D))
                hi = min(m0 + tile_m, N) if is_causal else N
                for n0 in range(0, hi, tile_n):
                    cols = np.arange(n0, min(n0 + tile_n, hi))
                    s = sm_scale * (qt @ k[b, g, cols].T)
                    if is_causal:
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m, s.max(axis=1))
                    with np.errstate(invalid="ignore"):
                        alpha = np.exp(m - m_new)
                    alpha = np.where(np.isneginf(m), 0.0, alpha)
                    p = np.exp(s - m_new[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, g, cols]
                    m = m_new
                O[b, h, rows] = acc / l[:, None]
                L[b, h, rows] = m + np.log(l)
    return O, L
