"""CPU float64 oracle for multi-head latent attention (MLA) decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite, the smoke check in the repository's entry module and the
CPU-baseline leg of the benchmark may import or call it.  It shares no code,
table or helper with the HIP library.

Definitions follow page "Attention Kernel 实现与正确性验证", section 2
(2.1 the absorption trick, 2.2 the PyTorch reference with its naive and
absorbed forms, 2.3 the DeepSeek-V3 shapes H=128, d_c=512, d_h_nope=d_v=128,
d_R=64).  Shapes:

    c_kv    [B, T, d_c]       compressed KV cache
    k_pe    [B, T, d_R]       rotary key part, shared by all heads
    q_nope  [B, H, S, d_nope]
    q_pe    [B, H, S, d_R]
    W_uk    [H, d_nope, d_c]  key up-projection
    W_uv    [H, d_v, d_c]     value up-projection

Naive form (the definition): per head h, K_nope = c_kv W_uk[h]^T,
V = c_kv W_uv[h]^T, K = [K_nope, k_pe], Q = [q_nope, q_pe],
out = softmax(Q K^T * sm_scale) V.  The page scales by 1/sqrt(d_nope + d_R).

Absorbed form: q_lat = [q_nope W_uk[h], q_pe] (d_c + d_R wide) and the
latent cache kv = [c_kv, k_pe]; scores q_lat kv^T equal Q K^T exactly, the
latent output out_lat = softmax(...) c_kv, and out = out_lat W_uv[h]^T.

Causal masking for S > 1 query tokens is bottom-right aligned (token s sits
at cache position s + T - S), the reading used for N_q < N_kv elsewhere.
Implementation shape: everything materialised per (b, h) in float64.
"""
from __future__ import annotations

import numpy as np


def _mask(S_, T, is_causal):
    if not is_causal:
        return None
    s = np.arange(S_)[:, None]
    j = np.arange(T)[None, :]
    return j > s + (T - S_)


def _softmax_rows(X):
    m = X.max(axis=1)
    E = np.exp(X - m[:, None])
    l = E.sum(axis=1)
    return E / l[:, None], m + np.log(l)


def mla_naive(c_kv, k_pe, q_nope, q_pe, W_uk, W_uv, *, is_causal: bool, sm_scale: float):
    """out [B, H, S, d_v] by reconstructing K and V per head (the definition)."""
    B, T, _ = c_kv.shape
    _, H, S_, _ = q_nope.shape
    d_v = W_uv.shape[1]
    if is_causal and S_ > T:
        raise ValueError("causal needs S <= T")
    mask = _mask(S_, T, is_causal)
    out = np.empty((B, H, S_, d_v))
    for b in range(B):
        for h in range(H):
            K = np.concatenate([c_kv[b] @ W_uk[h].T, k_pe[b]], axis=1)       # [T, d_nope + d_R]
            V = c_kv[b] @ W_uv[h].T                                          # [T, d_v]
            Q = np.concatenate([q_nope[b, h], q_pe[b, h]], axis=1)           # [S, d_nope + d_R]
            X = sm_scale * (Q @ K.T)
            if mask is not None:
                X = np.where(mask, -np.inf, X)
            P, _ = _softmax_rows(X)
            out[b, h] = P @ V
    return out


def mla_absorb_q(q_nope, q_pe, W_uk):
    """q_lat [B, H, S, d_c + d_R] = [q_nope W_uk[h], q_pe] per head."""
    return np.concatenate([np.einsum("bhsd,hdc->bhsc", q_nope, W_uk), q_pe], axis=-1)


def mla_latent_attention(q_lat, kv, d_c: int, *, is_causal: bool, sm_scale: float):
    """(out_lat [B, H, S, d_c], lse [B, H, S]) of the latent attention: scores
    q_lat kv^T over the whole latent row, values the first d_c columns of kv."""
    B, H, S_, _ = q_lat.shape
    T = kv.shape[1]
    if is_causal and S_ > T:
        raise ValueError("causal needs S <= T")
    mask = _mask(S_, T, is_causal)
    out = np.empty((B, H, S_, d_c))
    lse = np.empty((B, H, S_))
    for b in range(B):
        for h in range(H):
            X = sm_scale * (q_lat[b, h] @ kv[b].T)
            if mask is not None:
                X = np.where(mask, -np.inf, X)
            P, lse[b, h] = _softmax_rows(X)
            out[b, h] = P @ kv[b, :, :d_c]
    return out, lse


def mla_up_project(out_lat, W_uv):
    """out [B, H, S, d_v] = out_lat W_uv[h]^T per head."""
    return np.einsum("bhsc,hvc->bhsv", out_lat, W_uv)


def mla_absorbed(c_kv, k_pe, q_nope, q_pe, W_uk, W_uv, *, is_causal: bool, sm_scale: float):
    """The absorbed pipeline: absorb Q, latent attention, up-project."""
    q_lat = mla_absorb_q(q_nope, q_pe, W_uk)
    kv = np.concatenate([c_kv, k_pe], axis=-1)
    out_lat, _ = mla_latent_attention(q_lat, kv, c_kv.shape[-1], is_causal=is_causal,
                                      sm_scale=sm_scale)
    return mla_up_project(out_lat, W_uv)
