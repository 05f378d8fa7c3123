"""CPU float64 oracle for the attention backward pass: dQ, dK, dV.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite, the smoke check in the repository's entry module and the
CPU-baseline leg of the benchmark may import or call it.  It shares no code,
table or helper with the HIP library.

What it computes is the gradient of the scalar sum(dO * O) with respect to Q,
K and V, where O is the attention of the forward oracle (same head map, scale,
mask and alignment).  The method the pages give for it (page "Attention
Kernel 实现与正确性验证", section 1.1, third trick: the backward recomputes the
attention instead of storing S; page "Flash Attention 与 Kernel 优化", section
"Autograd 包装与反向传播": rebuild s = q k^T * scale, apply the causal mask,
rebuild p = softmax(s), then compute dv, dp, ds, dq, dk) is, for one batch
element b, query head h and kv head g:

    S   = sm_scale * Q K^T        (masked entries -inf)
    P   = softmax(S) row by row
    dV += P^T dO                  (summed over the query heads of kv head g)
    dP  = dO V^T
    Dl  = rowsum(dO * O)          ( = rowsum(P * dP) )
    dS  = P * (dP - Dl)
    dQ  = sm_scale * dS K
    dK += sm_scale * dS^T Q       (summed over the query heads of kv head g)

The gradient through the softmax, dS = P * (dP - rowsum(P * dP)), is the
Jacobian of the row softmax applied to dP; Dl is taken as rowsum(dO * O), which
equals rowsum(P * dP) because O = P V.  The forward hands q, k, v, the
log-sum-exp and o to the backward (page "Flash Attention 与 Kernel 优化",
"输出与保存状态": all five are kept in the autograd context), so o is an input
of the backward: with `out` given, Dl = rowsum(dO * out) uses it (a GPU
backward receives the bf16-rounded forward output); without it, O is
computed here, which gives the exact gradient.

Implementation shape: per (b, h) the full score matrix is materialised (so
inputs are limited to a few thousand rows and keys), in float64, with no
blocking.  `backward_rows` and `backward_keys` compute the same quantities for
chosen query rows (dQ) or chosen keys (dK, dV) of one head, taking query rows
in blocks of ROW_BLOCK, for inputs too large for the full matrix;
`backward_keys` can also sum over a subset of the query rows, so that a
caller may split the sum over rows across processes.
"""
from __future__ import annotations

import numpy as np

from .naive_attention import ROW_BLOCK, _check, kv_head


def _probs(q, k, b, h, g, rows, *, is_causal, sm_scale, off, keys=None):
    """Softmax rows P[rows, keys] of (b, h) (all keys when keys is None)."""
    N_kv = k.shape[2]
    S = sm_scale * (q[b, h, rows, :] @ k[b, g].T)            # [R, N_kv]
    if is_causal:
        S = np.where(np.arange(N_kv)[None, :] > rows[:, None] + off, -np.inf, S)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    P = E / E.sum(axis=1)[:, None]
    return P if keys is None else P[:, keys]


def attention_backward(q, k, v, dout, *, is_causal: bool, sm_scale: float, out=None):
    """(dQ [B,H_q,N_q,D], dK [B,H_kv,N_kv,D], dV [B,H_kv,N_kv,D]) in float64.

    out: optional forward output [B,H_q,N_q,D] used for Dl (see above)."""
    B, H_q, H_kv, N_q, N_kv, D = _check(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    if is_causal and N_q > N_kv:
        raise ValueError("causal attention needs N_q <= N_kv")
    off = N_kv - N_q if is_causal else 0
    dQ = np.zeros_like(q, dtype=np.float64)
    dK = np.zeros_like(k, dtype=np.float64)
    dV = np.zeros_like(v, dtype=np.float64)
    rows = np.arange(N_q)
    for b in range(B):
        for h in range(H_q):
            g = kv_head(h, H_q, H_kv)
            P = _probs(q, k, b, h, g, rows, is_causal=is_causal, sm_scale=sm_scale, off=off)
            dO = dout[b, h]
            O = P @ v[b, g] if out is None else out[b, h]
            dV[b, g] += P.T @ dO
            dP = dO @ v[b, g].T
            Dl = (dO * O).sum(axis=1)
            dS = P * (dP - Dl[:, None])
            dQ[b, h] = sm_scale * (dS @ k[b, g])
            dK[b, g] += sm_scale * (dS.T @ q[b, h])
    return dQ, dK, dV


def backward_rows(q, k, v, dout, b: int, h: int, rows, *, is_causal: bool, sm_scale: float,
                  out=None):
    """dQ[b, h, rows] ([len(rows), D], float64); out as in attention_backward."""
    B, H_q, H_kv, N_q, N_kv, D = _check(q, k, v)
    off = N_kv - N_q if is_causal else 0
    g = kv_head(h, H_q, H_kv)
    rows = np.asarray(rows, dtype=np.int64)
    res = np.empty((rows.size, D))
    for s in range(0, rows.size, ROW_BLOCK):
        r = rows[s:s + ROW_BLOCK]
        P = _probs(q, k, b, h, g, r, is_causal=is_causal, sm_scale=sm_scale, off=off)
        dO = dout[b, h, r]
        O = P @ v[b, g] if out is None else out[b, h, r]
        dP = dO @ v[b, g].T
        Dl = (dO * O).sum(axis=1)
        dS = P * (dP - Dl[:, None])
        res[s:s + ROW_BLOCK] = sm_scale * (dS @ k[b, g])
    return res


def backward_keys(q, k, v, dout, b: int, g: int, keys, *, is_causal: bool, sm_scale: float,
                  out=None, rows=None):
    """(dK[b, g, keys], dV[b, g, keys]) ([len(keys), D] each, float64), summed
    over the query heads of kv head g and all their rows; out as in
    attention_backward.  rows (optional): sum over these query rows only (of
    every head of the group), the part of the sum they contribute; the
    default is every row."""
    B, H_q, H_kv, N_q, N_kv, D = _check(q, k, v)
    off = N_kv - N_q if is_causal else 0
    keys = np.asarray(keys, dtype=np.int64)
    rows = np.arange(N_q) if rows is None else np.asarray(rows, dtype=np.int64)
    dK = np.zeros((keys.size, D))
    dV = np.zeros((keys.size, D))
    heads = [h for h in range(H_q) if kv_head(h, H_q, H_kv) == g]
    for h in heads:
        for s in range(0, rows.size, ROW_BLOCK):
            r = rows[s:s + ROW_BLOCK]
            P = _probs(q, k, b, h, g, r, is_causal=is_causal, sm_scale=sm_scale, off=off)
            dO = dout[b, h, r]
            O = P @ v[b, g] if out is None else out[b, h, r]
            Dl = (dO * O).sum(axis=1)
            Pk = P[:, keys]
            dPk = dO @ v[b, g, keys].T
            dSk = Pk * (dPk - Dl[:, None])
            dV += Pk.T @ dO
            dK += sm_scale * (dSk.T @ q[b, h, r])
    return dK, dV
