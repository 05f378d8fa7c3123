"""Checks that pin the MLA oracle to facts other than itself.

Each check takes a namespace `ora` with mla_naive, mla_absorbed, mla_absorb_q,
mla_latent_attention, mla_up_project (possibly a mutant) and
attention_forward (the pinned forward oracle) and raises AssertionError on
failure.

Pins used:
  * library: the naive form against PyTorch's scaled_dot_product_attention in
    float64 on explicitly reconstructed K and V (with the lower-right causal
    bias for S > 1);
  * the absorption identity of the page's section 2.1: absorbed == naive;
  * special case: the latent attention equals the pinned forward oracle with
    one kv head whose values are the whole latent row, truncated to d_c;
  * closed forms: one cached token (out = its value), zero scale (mean of the
    visible values), identity projections.
"""
from __future__ import annotations

import numpy as np

TOL = 1e-10


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * (1 + np.max(np.abs(b), initial=0.0)), f"{what}: max err {err}"


def _mla_inputs(B, H, S, T, d_c, d_nope, d_r, d_v, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, T, d_c)), r.standard_normal((B, T, d_r)),
            r.standard_normal((B, H, S, d_nope)), r.standard_normal((B, H, S, d_r)),
            r.standard_normal((H, d_nope, d_c)) / np.sqrt(d_c),
            r.standard_normal((H, d_v, d_c)) / np.sqrt(d_c))


SHAPES = [(1, 4, 1, 13, 16, 8, 4, 8, 1, False), (2, 3, 3, 11, 12, 6, 4, 5, 2, True),
          (1, 2, 5, 5, 8, 8, 2, 8, 3, True), (1, 2, 2, 9, 8, 4, 2, 6, 4, False)]


def pin_mla_naive_vs_torch_sdpa(ora):
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    for (B, H, S, T, d_c, d_nope, d_r, d_v, seed, causal) in SHAPES:
        c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = _mla_inputs(B, H, S, T, d_c, d_nope, d_r, d_v, seed)
        sc = 1.0 / np.sqrt(d_nope + d_r)
        K = np.concatenate([np.einsum("btc,hdc->bhtd", c_kv, W_uk),
                            np.broadcast_to(k_pe[:, None], (B, H, T, d_r))], axis=-1)
        V = np.einsum("btc,hvc->bhtv", c_kv, W_uv)
        Q = np.concatenate([q_nope, q_pe], axis=-1)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
        if causal and S != T:
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(S, T), scale=sc)
        else:
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc)
        got = ora.mla_naive(c_kv, k_pe, q_nope, q_pe, W_uk, W_uv, is_causal=causal, sm_scale=sc)
        _close(got, ref.numpy(), what="naive vs sdpa")


def pin_mla_absorbed_equals_naive(ora):
    for (B, H, S, T, d_c, d_nope, d_r, d_v, seed, causal) in SHAPES:
        args = _mla_inputs(B, H, S, T, d_c, d_nope, d_r, d_v, seed + 10)
        sc = 1.0 / np.sqrt(d_nope + d_r)
        _close(ora.mla_absorbed(*args, is_causal=causal, sm_scale=sc),
               ora.mla_naive(*args, is_causal=causal, sm_scale=sc), what="absorbed vs naive")


def pin_mla_latent_is_mqa_attention(ora):
    for (B, H, S, T, d_c, d_nope, d_r, d_v, seed, causal) in SHAPES:
        r = np.random.default_rng(seed + 20)
        q_lat = r.standard_normal((B, H, S, d_c + d_r))
        kv = r.standard_normal((B, T, d_c + d_r))
        sc = 0.3
        out, lse = ora.mla_latent_attention(q_lat, kv, d_c, is_causal=causal, sm_scale=sc)
        O, L = ora.attention_forward(q_lat, kv[:, None], kv[:, None], is_causal=causal, sm_scale=sc)
        _close(out, O[..., :d_c], what="latent vs attention")
        _close(lse, L, what="latent lse")


def pin_mla_one_token(ora):
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = _mla_inputs(2, 3, 1, 1, 8, 4, 2, 5, 31)
    out = ora.mla_absorbed(c_kv, k_pe, q_nope, q_pe, W_uk, W_uv, is_causal=True, sm_scale=0.4)
    _close(out, np.einsum("btc,hvc->bhtv", c_kv[:, :1], W_uv), what="one token")
    q_lat = ora.mla_absorb_q(q_nope, q_pe, W_uk)
    kv = np.concatenate([c_kv, k_pe], axis=-1)
    o, l = ora.mla_latent_attention(q_lat, kv, 8, is_causal=False, sm_scale=0.4)
    _close(o, np.broadcast_to(c_kv[:, None], o.shape), what="one token latent")
    _close(l, 0.4 * np.einsum("bhsc,btc->bhs", q_lat, kv), what="one token lse")


def pin_mla_zero_scale(ora):
    r = np.random.default_rng(41)
    q_lat = r.standard_normal((1, 2, 3, 10))
    kv = r.standard_normal((1, 7, 10))
    for causal in (False, True):
        o, l = ora.mla_latent_attention(q_lat, kv, 8, is_causal=causal, sm_scale=0.0)
        for s in range(3):
            n = s + 5 if causal else 7
            _close(o[0, :, s], np.broadcast_to(kv[0, :n, :8].mean(axis=0), (2, 8)), what="scale0")
            _close(l[0, :, s], np.full(2, np.log(n)), what="scale0 lse")


def pin_mla_identity_projections(ora):
    r = np.random.default_rng(51)
    q_nope = r.standard_normal((1, 2, 1, 6))
    q_pe = r.standard_normal((1, 2, 1, 3))
    eye = np.broadcast_to(np.eye(6), (2, 6, 6)).copy()
    _close(ora.mla_absorb_q(q_nope, q_pe, eye), np.concatenate([q_nope, q_pe], -1), what="absorb I")
    x = r.standard_normal((1, 2, 4, 6))
    _close(ora.mla_up_project(x, eye), x, what="up I")
    W = r.standard_normal((2, 3, 6))
    _close(ora.mla_up_project(x, W)[0, 1, 2], W[1] @ x[0, 1, 2], what="up row")
    Wk = r.standard_normal((2, 6, 5))
    _close(ora.mla_absorb_q(q_nope, q_pe, Wk)[0, 1, 0, :5], q_nope[0, 1, 0] @ Wk[1], what="absorb row")


PINS_MLA = [pin_mla_naive_vs_torch_sdpa, pin_mla_absorbed_equals_naive, pin_mla_latent_is_mqa_attention,
            pin_mla_one_token, pin_mla_zero_scale, pin_mla_identity_projections]
