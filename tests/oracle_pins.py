"""Checks that pin the CPU oracle to facts other than itself.

Each check takes an oracle namespace `ora` (with attention_forward,
attention_rows, kv_head and merge_partials) and raises AssertionError on failure.  They are
run against the real oracle (all must pass) and against mutants of it with a
planted mistake (at least one must fail), so each pin is shown to bite.

Pins used:
  * brute force: scalar loops with exactly-rounded sums (math.fsum) on tiny
    inputs, independent of NumPy;
  * closed forms: N = 1, two keys, sm_scale = 0, identical keys, causal row 0;
  * invariants: rows of the softmax sum to 1, output in the convex hull of
    the visible values, causal prefix, joint key/value permutation, shift of
    every key by a common vector, large scores without overflow;
  * head map: both printed formulas agree, and GQA equals MHA on repeated K/V;
  * library special cases: scipy logsumexp of the scores, and PyTorch's
    scaled_dot_product_attention in float64 on the CPU (with its lower-right
    causal bias for N_q < N_kv);
  * fewer query rows than keys: brute force, the suffix of square causal
    attention, decode (one row sees every key);
  * merge of partial results: disjoint key splits merged through their LSEs
    equal attention over all keys.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(B, H_q, H_kv, N, D, seed, scale=1.0):
    return (_rand((B, H_q, N, D), seed, scale), _rand((B, H_kv, N, D), seed + 1, scale),
            _rand((B, H_kv, N, D), seed + 2, scale))


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * (1 + np.max(np.abs(b), initial=0.0)), f"{what}: max err {err}"


def _brute(q, k, v, is_causal, sm_scale):
    """Scalar-loop attention with exactly rounded sums; tiny inputs only.

    With fewer query rows than keys, causal row i sees keys 0..i + N_kv - N_q
    (the last query row sees every key)."""
    B, H_q, N, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    off = N_kv - N
    G = H_q // H_kv
    O = np.zeros((B, H_q, N, D))
    L = np.zeros((B, H_q, N))
    for b in range(B):
        for h in range(H_q):
            g = h // G
            for i in range(N):
                keys = range(i + off + 1) if is_causal else range(N_kv)
                s = [sm_scale * math.fsum(q[b, h, i, d] * k[b, g, j, d] for d in range(D))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(w[t] * v[b, g, j, d] for t, j in enumerate(keys)) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


# ---------------------------------------------------------------- brute force
def pin_brute_force_tiny(ora):
    for (B, H_q, H_kv, N, D, causal, seed) in [
        (1, 2, 2, 5, 3, False, 11), (2, 4, 2, 7, 4, True, 12), (1, 3, 1, 6, 2, True, 13),
        (1, 4, 4, 9, 5, False, 14), (2, 2, 1, 4, 8, False, 15),
    ]:
        q, k, v = _qkv(B, H_q, H_kv, N, D, seed)
        sc = 0.7
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        Ob, Lb = _brute(q, k, v, causal, sc)
        _close(O, Ob, what="brute O")
        _close(L, Lb, what="brute LSE")


def pin_brute_force_rect(ora):
    """Fewer query rows than keys (prefill against a cache, decode)."""
    rng = np.random.default_rng(16)
    for (B, H_q, H_kv, N_q, N_kv, D, causal) in [
        (1, 2, 1, 3, 8, 4, True), (2, 4, 2, 1, 9, 3, True), (1, 2, 2, 4, 7, 5, False),
        (1, 3, 1, 1, 5, 2, False), (1, 2, 1, 6, 6, 3, True),
    ]:
        q = rng.standard_normal((B, H_q, N_q, D))
        k = rng.standard_normal((B, H_kv, N_kv, D))
        v = rng.standard_normal((B, H_kv, N_kv, D))
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=0.6)
        Ob, Lb = _brute(q, k, v, causal, 0.6)
        _close(O, Ob, what="brute rect O")
        _close(L, Lb, what="brute rect LSE")


# ---------------------------------------------------------------- closed forms
def pin_single_key(ora):
    """N = 1: the only key gets weight 1, LSE is its scaled score."""
    q, k, v = _qkv(2, 4, 2, 1, 16, 21)
    sc = 0.31
    for causal in (False, True):
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        for b in range(2):
            for h in range(4):
                g = h // 2
                _close(O[b, h, 0], v[b, g, 0], what="N=1 O")
                _close(L[b, h, 0], sc * math.fsum(q[b, h, 0] * k[b, g, 0]), what="N=1 LSE")


def pin_two_keys(ora):
    """N = 2, non-causal: weight of key 0 is the logistic of s0 - s1."""
    q, k, v = _qkv(1, 2, 1, 2, 8, 31)
    sc = 0.9
    O, L = ora.attention_forward(q, k, v, is_causal=False, sm_scale=sc)
    for h in range(2):
        for i in range(2):
            s0 = sc * math.fsum(q[0, h, i] * k[0, 0, 0])
            s1 = sc * math.fsum(q[0, h, i] * k[0, 0, 1])
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            _close(O[0, h, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], what="2-key O")
            _close(L[0, h, i], max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))),
                   what="2-key LSE")


def pin_zero_scale(ora):
    """sm_scale = 0: uniform weights over the visible keys."""
    q, k, v = _qkv(1, 2, 2, 9, 4, 41)
    for causal in (False, True):
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=0.0)
        for h in range(2):
            for i in range(9):
                n = i + 1 if causal else 9
                _close(O[0, h, i], v[0, h, :n].mean(axis=0), what="scale0 O")
                _close(L[0, h, i], math.log(n), what="scale0 LSE")


def pin_identical_keys(ora):
    """All keys equal: O is the mean of the visible V, LSE = s + ln(#visible)."""
    q, k, v = _qkv(1, 2, 1, 8, 6, 51)
    k[:] = k[:, :, :1, :]
    sc = 0.5
    for causal in (False, True):
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        for h in range(2):
            for i in range(8):
                n = i + 1 if causal else 8
                s = sc * math.fsum(q[0, h, i] * k[0, 0, 0])
                _close(O[0, h, i], v[0, 0, :n].mean(axis=0), what="ident O")
                _close(L[0, h, i], s + math.log(n), what="ident LSE")


def pin_causal_row0(ora):
    """Causal row 0 sees only key 0."""
    q, k, v = _qkv(2, 4, 4, 12, 8, 61)
    sc = 0.8
    O, L = ora.attention_forward(q, k, v, is_causal=True, sm_scale=sc)
    for b in range(2):
        for h in range(4):
            _close(O[b, h, 0], v[b, h, 0], what="row0 O")
            _close(L[b, h, 0], sc * math.fsum(q[b, h, 0] * k[b, h, 0]), what="row0 LSE")


# ---------------------------------------------------------------- invariants
def _scores(q, k, b, h, g, sc):
    N = q.shape[2]
    return np.array([[sc * math.fsum(q[b, h, i] * k[b, g, j]) for j in range(N)]
                     for i in range(N)])


def pin_rows_sum_to_one(ora):
    """sum_j exp(S_ij - LSE_i) = 1 over the visible keys."""
    q, k, v = _qkv(1, 4, 2, 10, 5, 71)
    sc = 0.6
    for causal in (False, True):
        _, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        for h in range(4):
            S = _scores(q, k, 0, h, h // 2, sc)
            for i in range(10):
                n = i + 1 if causal else 10
                _close(math.fsum(math.exp(S[i, j] - L[0, h, i]) for j in range(n)), 1.0,
                       what="row sum")


def pin_convex_hull(ora):
    """Each output lies inside the box spanned by the visible V rows."""
    q, k, v = _qkv(1, 2, 2, 16, 4, 81, scale=2.0)
    for causal in (False, True):
        O, _ = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=1.0)
        for h in range(2):
            for i in range(16):
                n = i + 1 if causal else 16
                lo = v[0, h, :n].min(axis=0) - 1e-12
                hi = v[0, h, :n].max(axis=0) + 1e-12
                assert np.all(O[0, h, i] >= lo) and np.all(O[0, h, i] <= hi), "outside hull"


def pin_causal_prefix(ora):
    """Causal row i equals non-causal attention over keys 0..i."""
    q, k, v = _qkv(1, 2, 1, 11, 4, 91)
    sc = 0.7
    O, L = ora.attention_forward(q, k, v, is_causal=True, sm_scale=sc)
    for i in range(11):
        Op, Lp = ora.attention_forward(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1],
                                       is_causal=False, sm_scale=sc)
        _close(O[:, :, i], Op[:, :, i], what="prefix O")
        _close(L[:, :, i], Lp[:, :, i], what="prefix LSE")


def pin_permutation(ora):
    """Non-causal output is invariant to a joint permutation of K and V rows."""
    q, k, v = _qkv(1, 2, 2, 13, 4, 101)
    perm = np.random.default_rng(5).permutation(13)
    O, L = ora.attention_forward(q, k, v, is_causal=False, sm_scale=0.9)
    Op, Lp = ora.attention_forward(q, k[:, :, perm], v[:, :, perm], is_causal=False,
                                   sm_scale=0.9)
    _close(O, Op, what="perm O")
    _close(L, Lp, what="perm LSE")


def pin_key_shift(ora):
    """Adding c to every key shifts row i's scores by sm_scale*q_i.c: O unchanged,
    LSE moves by that amount."""
    q, k, v = _qkv(1, 2, 2, 9, 4, 111)
    c = _rand((4,), 7, 3.0)
    sc = 0.4
    for causal in (False, True):
        O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        O2, L2 = ora.attention_forward(q, k + c, v, is_causal=causal, sm_scale=sc)
        _close(O2, O, tol=1e-11, what="shift O")
        _close(L2, L + sc * np.einsum("bhnd,d->bhn", q, c), tol=1e-11, what="shift LSE")


def pin_large_scores(ora):
    """Scores in the thousands must not overflow: max subtraction is required."""
    q, k, v = _qkv(1, 1, 1, 6, 4, 121)
    k[0, 0, 3] = q[0, 0, 5] * 400.0          # key 3 dominates row 5 by far
    O, L = ora.attention_forward(q, k, v, is_causal=False, sm_scale=1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), "overflow"
    _close(O[0, 0, 5], v[0, 0, 3], tol=1e-9, what="dominant key")


def pin_causal_suffix(ora):
    """N_q < N_kv causal rows are the last N_q rows of square causal attention
    whose queries end with them (the rect case reduces to the square one)."""
    q, k, v = _qkv(1, 2, 2, 10, 4, 161)
    sc = 0.8
    O, L = ora.attention_forward(q, k, v, is_causal=True, sm_scale=sc)
    for n_q in (1, 3, 9):
        Os, Ls = ora.attention_forward(q[:, :, 10 - n_q:], k, v, is_causal=True, sm_scale=sc)
        _close(Os, O[:, :, 10 - n_q:], what="suffix O")
        _close(Ls, L[:, :, 10 - n_q:], what="suffix LSE")


def pin_decode_sees_all_keys(ora):
    """A single query row with the causal flag attends to every key."""
    q, k, v = _qkv(2, 4, 1, 1, 4, 171)
    k = _rand((2, 1, 13, 4), 172)
    v = _rand((2, 1, 13, 4), 173)
    Oc, Lc = ora.attention_forward(q, k, v, is_causal=True, sm_scale=0.5)
    On, Ln = ora.attention_forward(q, k, v, is_causal=False, sm_scale=0.5)
    _close(Oc, On, what="decode O")
    _close(Lc, Ln, what="decode LSE")


def pin_merge_partials(ora):
    """Attention over disjoint key subsets, merged through the LSEs, equals
    attention over their union; an empty subset (lse = -inf, O = 0) adds
    nothing; LSE values in the thousands do not overflow the merge."""
    q, k, v = _qkv(1, 2, 1, 5, 4, 181)
    k = _rand((1, 1, 23, 4), 182)
    v = _rand((1, 1, 23, 4), 183)
    for sc in (0.7, 300.0):
        O, L = ora.attention_forward(q, k, v, is_causal=False, sm_scale=sc)
        cuts = [0, 6, 6, 17, 23]                       # one empty split
        os_, ls_ = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if a == b:
                os_.append(np.zeros_like(O))
                ls_.append(np.full_like(L, -np.inf))
            else:
                Op, Lp = ora.attention_forward(q, k[:, :, a:b], v[:, :, a:b], is_causal=False,
                                               sm_scale=sc)
                os_.append(Op)
                ls_.append(Lp)
        with np.errstate(over="raise"):
            Om, Lm = ora.merge_partials(np.stack(os_), np.stack(ls_))
        _close(Om, O, tol=1e-11, what="merged O")
        _close(Lm, L, tol=1e-11, what="merged LSE")


# ---------------------------------------------------------------- head map
def pin_head_map(ora):
    """Both printed GQA formulas agree on every divisible pair up to 128 heads."""
    for H_q in range(1, 129):
        for H_kv in range(1, H_q + 1):
            if H_q % H_kv:
                continue
            G = H_q // H_kv
            for h in range(H_q):
                assert ora.kv_head(h, H_q, H_kv) == h // G, (h, H_q, H_kv)


def pin_gqa_equals_repeated_mha(ora):
    """GQA on [B,H_kv,...] K/V equals MHA on K/V repeated G times per kv head."""
    for (H_q, H_kv) in [(8, 2), (6, 3), (4, 1)]:
        q, k, v = _qkv(2, H_q, H_kv, 7, 4, 131 + H_q)
        G = H_q // H_kv
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        for causal in (False, True):
            O, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=0.5)
            Or, Lr = ora.attention_forward(q, kr, vr, is_causal=causal, sm_scale=0.5)
            assert np.array_equal(O, Or) and np.array_equal(L, Lr), "GQA != repeated MHA"


# ---------------------------------------------------------------- libraries
def pin_scipy_logsumexp(ora):
    from scipy.special import logsumexp
    q, k, v = _qkv(1, 2, 1, 12, 6, 141)
    sc = 0.45
    for causal in (False, True):
        _, L = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        for h in range(2):
            S = _scores(q, k, 0, h, 0, sc)
            for i in range(12):
                n = i + 1 if causal else 12
                _close(L[0, h, i], logsumexp(S[i, :n]), what="logsumexp")


def pin_torch_sdpa(ora):
    import torch
    import torch.nn.functional as F
    for (B, H_q, H_kv, N, D, causal, seed) in [(1, 4, 4, 33, 16, False, 151),
                                               (2, 8, 2, 40, 8, True, 152),
                                               (1, 4, 1, 17, 32, True, 153)]:
        q, k, v = _qkv(B, H_q, H_kv, N, D, seed)
        sc = 1.0 / math.sqrt(D)
        G = H_q // H_kv
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.repeat(k, G, axis=1)),
            torch.from_numpy(np.repeat(v, G, axis=1)), is_causal=causal, scale=sc).numpy()
        O, _ = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=sc)
        _close(O, ref, what="sdpa")


def pin_torch_sdpa_lower_right(ora):
    """N_q != N_kv against PyTorch: plain non-causal, and causal through its
    bottom-right (lower-right) causal bias."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    rng = np.random.default_rng(191)
    for (N_q, N_kv, causal) in [(7, 30, False), (30, 7, False), (7, 30, True), (1, 19, True)]:
        q = rng.standard_normal((1, 2, N_q, 8))
        k = rng.standard_normal((1, 2, N_kv, 8))
        v = rng.standard_normal((1, 2, N_kv, 8))
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        if causal:
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(N_q, N_kv),
                                                 scale=0.3)
        else:
            ref = F.scaled_dot_product_attention(tq, tk, tv, scale=0.3)
        O, _ = ora.attention_forward(q, k, v, is_causal=causal, sm_scale=0.3)
        _close(O, ref.numpy(), what="sdpa lower-right")


PINS = [
    pin_brute_force_tiny, pin_single_key, pin_two_keys, pin_zero_scale, pin_identical_keys,
    pin_causal_row0, pin_rows_sum_to_one, pin_convex_hull, pin_causal_prefix,
    pin_permutation, pin_key_shift, pin_large_scores, pin_head_map,
    pin_gqa_equals_repeated_mha, pin_scipy_logsumexp, pin_torch_sdpa,
    pin_brute_force_rect, pin_causal_suffix, pin_decode_sees_all_keys, pin_merge_partials,
    pin_torch_sdpa_lower_right,
]
