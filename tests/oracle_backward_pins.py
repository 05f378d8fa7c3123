"""Checks that pin the backward oracle (dQ, dK, dV) to facts other than itself.

Each check takes a namespace `ora` with attention_backward, backward_rows,
backward_keys (the backward oracle, possibly a mutant) and attention_forward
(the pinned forward oracle), and raises AssertionError on failure.

Pins used:
  * finite differences: central differences of sum(dO * O) through the forward
    oracle, element by element, on tiny inputs (square, rectangular, causal,
    GQA);
  * library: PyTorch autograd through scaled_dot_product_attention in float64
    on the CPU (K/V repeated per group, gradients summed back; the lower-right
    causal bias for N_q < N_kv), for all three oracle entry points;
  * closed forms: one key (dQ = dK = 0, dV = summed dO), zero scale (dQ = dK = 0,
    dV = dO averaged over each row's visible keys), identical keys (dQ = 0);
  * invariant: the key gradients of a kv head sum to zero (softmax rows are
    invariant to a common shift of all keys);
  * head map: GQA gradients equal MHA gradients on repeated K/V, summed back;
  * the forward output as an input: the exact output changes nothing, and a
    perturbed one moves dQ by the closed-form amount and leaves dV unchanged;
  * key gradients over a subset of query rows: the parts over a partition of
    the rows sum to the key gradients of attention_backward, and the part of
    a single row is the outer-product formula written out for that row.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-10


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * (1 + np.max(np.abs(b), initial=0.0)), f"{what}: max err {err}"


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _inputs(B, H_q, H_kv, N_q, N_kv, D, seed):
    return (_rand((B, H_q, N_q, D), seed), _rand((B, H_kv, N_kv, D), seed + 1),
            _rand((B, H_kv, N_kv, D), seed + 2), _rand((B, H_q, N_q, D), seed + 3))


def pin_bwd_finite_differences(ora):
    eps = 1e-5
    for (B, H_q, H_kv, N_q, N_kv, D, causal, seed) in [
        (1, 2, 1, 3, 5, 3, True, 11), (1, 2, 2, 4, 4, 2, False, 12), (1, 3, 1, 4, 4, 2, True, 13),
        (1, 2, 1, 1, 6, 3, True, 14), (1, 1, 1, 5, 3, 2, False, 15),
    ]:
        q, k, v, dO = _inputs(B, H_q, H_kv, N_q, N_kv, D, seed)
        sc = 0.8

        def loss(q_, k_, v_):
            O, _ = ora.attention_forward(q_, k_, v_, is_causal=causal, sm_scale=sc)
            return float(np.sum(dO * O))

        dQ, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=sc)
        for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            _close(g, fd, tol=1e-7, what=f"FD d{name} {causal} {N_q}x{N_kv}")


def _torch_grads(q, k, v, dO, causal, sc):
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    H_q, H_kv = q.shape[1], k.shape[1]
    G = H_q // H_kv
    tq = torch.from_numpy(q).requires_grad_(True)
    tk = torch.from_numpy(k).requires_grad_(True)
    tv = torch.from_numpy(v).requires_grad_(True)
    kr = tk.repeat_interleave(G, dim=1)
    vr = tv.repeat_interleave(G, dim=1)
    N_q, N_kv = q.shape[2], k.shape[2]
    if causal and N_q != N_kv:
        o = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=causal_lower_right(N_q, N_kv),
                                           scale=sc)
    else:
        o = F.scaled_dot_product_attention(tq, kr, vr, is_causal=causal, scale=sc)
    o.backward(torch.from_numpy(dO))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_bwd_torch_autograd(ora):
    for (B, H_q, H_kv, N_q, N_kv, D, causal, seed) in [
        (2, 4, 2, 17, 17, 8, True, 21), (1, 4, 4, 9, 23, 16, False, 22),
        (1, 6, 2, 7, 30, 8, True, 23), (1, 3, 1, 1, 19, 8, True, 24),
    ]:
        q, k, v, dO = _inputs(B, H_q, H_kv, N_q, N_kv, D, seed)
        sc = 1.0 / math.sqrt(D)
        tq, tk, tv = _torch_grads(q, k, v, dO, causal, sc)
        dQ, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=sc)
        _close(dQ, tq, what="torch dQ")
        _close(dK, tk, what="torch dK")
        _close(dV, tv, what="torch dV")
        rows = np.array([0, N_q - 1, N_q // 2])
        for h in (0, H_q - 1):
            _close(ora.backward_rows(q, k, v, dO, B - 1, h, rows, is_causal=causal, sm_scale=sc),
                   tq[B - 1, h, rows], what="torch dQ rows")
        keys = np.array([0, N_kv - 1, N_kv // 3])
        for g in range(H_kv):
            bk, bv = ora.backward_keys(q, k, v, dO, 0, g, keys, is_causal=causal, sm_scale=sc)
            _close(bk, tk[0, g, keys], what="torch dK keys")
            _close(bv, tv[0, g, keys], what="torch dV keys")


def pin_bwd_single_key(ora):
    q, k, v, dO = _inputs(2, 4, 2, 3, 1, 8, 31)
    dQ, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=False, sm_scale=0.7)
    _close(dQ, np.zeros_like(dQ), what="1-key dQ")
    _close(dK, np.zeros_like(dK), what="1-key dK")
    for b in range(2):
        for g in range(2):
            _close(dV[b, g, 0], dO[b, 2 * g:2 * g + 2].sum(axis=(0, 1)), what="1-key dV")


def pin_bwd_zero_scale(ora):
    q, k, v, dO = _inputs(1, 2, 1, 6, 6, 4, 41)
    for causal in (False, True):
        dQ, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.0)
        _close(dQ, np.zeros_like(dQ), what="scale0 dQ")
        _close(dK, np.zeros_like(dK), what="scale0 dK")
        for j in range(6):
            exp = sum(dO[0, h, i] / ((i + 1) if causal else 6)
                      for h in range(2) for i in range(6) if (not causal or j <= i))
            _close(dV[0, 0, j], exp, what="scale0 dV")


def pin_bwd_identical_keys(ora):
    q, k, v, dO = _inputs(1, 2, 1, 7, 7, 5, 51)
    k[:] = k[:, :, :1]
    for causal in (False, True):
        dQ, _, _ = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.6)
        _close(dQ, np.zeros_like(dQ), what="identical keys dQ")


def pin_bwd_key_grads_sum_to_zero(ora):
    q, k, v, dO = _inputs(2, 4, 2, 9, 12, 6, 61)
    for causal in (False, True):
        _, dK, _ = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.9)
        _close(dK.sum(axis=2), np.zeros((2, 2, 6)), what="sum_j dK_j")


def pin_bwd_gqa_equals_repeated(ora):
    q, k, v, dO = _inputs(1, 6, 2, 8, 8, 4, 71)
    for causal in (False, True):
        dQ, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.5)
        kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
        dQr, dKr, dVr = ora.attention_backward(q, kr, vr, dO, is_causal=causal, sm_scale=0.5)
        _close(dQ, dQr, tol=1e-13, what="gqa dQ")
        _close(dK, dKr.reshape(1, 2, 3, 8, 4).sum(axis=2), tol=1e-13, what="gqa dK")
        _close(dV, dVr.reshape(1, 2, 3, 8, 4).sum(axis=2), tol=1e-13, what="gqa dV")


def pin_bwd_supplied_exact_output(ora):
    """Handing the backward the exact forward output changes nothing; a
    perturbed output moves dQ by exactly -scale * (dO . delta) * (P K) per row."""
    q, k, v, dO = _inputs(1, 4, 2, 11, 14, 6, 81)
    for causal in (False, True):
        O, _ = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=0.7)
        ref = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.7)
        got = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.7, out=O)
        for a, b_ in zip(got, ref):
            _close(a, b_, tol=1e-13, what="supplied O")
        dl = _rand(O.shape, 82, 1e-3)
        dQ2, dK2, dV2 = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.7,
                                               out=O + dl)
        _close(dV2, ref[2], tol=1e-13, what="dV independent of O")
        # dS changes by -P * delta_i with delta_i = dO_i . dl_i, so dQ_i by -0.7 delta_i (P K)_i;
        # (P K)_i is attention with K as the values
        shift = np.einsum("bhnd,bhnd->bhn", dO, dl)
        PK, _ = ora.attention_forward(q, k, k, is_causal=causal, sm_scale=0.7)
        _close(dQ2, ref[0] - 0.7 * shift[..., None] * PK, tol=1e-12, what="dQ shift")
        rows = np.array([0, 10])
        _close(ora.backward_rows(q, k, v, dO, 0, 1, rows, is_causal=causal, sm_scale=0.7, out=O + dl),
               dQ2[0, 1, rows], what="rows with out")
        keys = np.array([0, 13])
        bk, _ = ora.backward_keys(q, k, v, dO, 0, 1, keys, is_causal=causal, sm_scale=0.7, out=O + dl)
        _close(bk, dK2[0, 1, keys], what="keys with out")


def pin_bwd_keys_row_partition(ora):
    """dK, dV of chosen keys summed over a partition of the query rows equal
    the full gradients; one row's part is its own rank-one term, written out
    per element: dV_j = sum_h P_hj dO_h, dK_j = scale sum_h P_hj (dP_hj - Dl_h) q_h."""
    q, k, v, dO = _inputs(1, 4, 2, 9, 13, 5, 91)
    keys = np.array([0, 4, 12])
    for causal in (False, True):
        _, dK, dV = ora.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.7)
        parts = [np.array([0, 3, 8]), np.array([1, 2]), np.array([4, 5, 6, 7])]
        got = [ora.backward_keys(q, k, v, dO, 0, 1, keys, is_causal=causal, sm_scale=0.7, rows=r)
               for r in parts]
        _close(sum(g_[0] for g_ in got), dK[0, 1, keys], what="row partition dK")
        _close(sum(g_[1] for g_ in got), dV[0, 1, keys], what="row partition dV")
        i = 6
        bk, bv = ora.backward_keys(q, k, v, dO, 0, 1, keys, is_causal=causal, sm_scale=0.7,
                                   rows=np.array([i]))
        off = 13 - 9 if causal else 0
        ek, ev = np.zeros_like(bk), np.zeros_like(bv)
        for h in (2, 3):  # the query heads of kv head 1
            s_ = [0.7 * sum(q[0, h, i, d] * k[0, 1, j, d] for d in range(5)) for j in range(13)]
            vis = [j for j in range(13) if not causal or j <= i + off]
            m = max(s_[j] for j in vis)
            z = sum(math.exp(s_[j] - m) for j in vis)
            p = [math.exp(s_[j] - m) / z if j in vis else 0.0 for j in range(13)]
            dp = [sum(dO[0, h, i, d] * v[0, 1, j, d] for d in range(5)) for j in range(13)]
            dl = sum(p[j] * dp[j] for j in range(13))
            for n, j in enumerate(keys):
                ev[n] += p[j] * dO[0, h, i]
                ek[n] += 0.7 * p[j] * (dp[j] - dl) * q[0, h, i]
        _close(bk, ek, what="one row's dK part")
        _close(bv, ev, what="one row's dV part")


PINS_BWD = [
    pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_single_key, pin_bwd_zero_scale,
    pin_bwd_identical_keys, pin_bwd_key_grads_sum_to_zero, pin_bwd_gqa_equals_repeated,
    pin_bwd_supplied_exact_output, pin_bwd_keys_row_partition,
]
