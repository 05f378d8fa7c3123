"""GPU parity: the HIP attention forward against the float64 CPU oracle.

Every case draws seeded bf16 inputs, runs attn_fwd through the C ABI (via the
ctypes binding) and compares element by element with the oracle on the same
bf16 values.  Tolerances: |O - O_ref| <= 2e-2 + 2e-2 |O_ref| (the bf16
atol = rtol = 2e-2 of the page "Attention Kernel 实现与正确性验证", section 1.3)
and |LSE - LSE_ref| <= 1e-3; no NaN or Inf anywhere.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

O_ATOL = 2e-2
O_RTOL = 2e-2
LSE_ATOL = 1e-3
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_02_amd as m
    m.load_library()
    return m


def _run(ea, q, k, v, causal, scale, poison=True):
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H_q, N, D = q.shape
    out = torch.empty((B, H_q, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H_q, N), dtype=torch.float32, device=dev)
    if poison:
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    ea.attn_fwd(qd, kd, vd, out, lse, is_causal=causal, sm_scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(o_gpu, l_gpu, O_ref, L_ref, what=""):
    o = o_gpu.to(torch.float64).numpy() if isinstance(o_gpu, torch.Tensor) else o_gpu
    l = l_gpu.to(torch.float64).numpy() if isinstance(l_gpu, torch.Tensor) else l_gpu
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(l)), f"{what}: non-finite LSE"
    err_o = np.abs(o - O_ref)
    bound = O_ATOL + O_RTOL * np.abs(O_ref)
    bad = err_o > bound
    err_l = np.abs(l - L_ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} O elements out of tolerance; "
                           f"max abs err {err_o.max():.3e} at {np.unravel_index(err_o.argmax(), err_o.shape)}")
    assert err_l.max(initial=0.0) <= LSE_ATOL, f"{what}: max LSE err {err_l.max():.3e}"
    return float(err_o.max(initial=0.0)), float(err_l.max(initial=0.0))


def _full_case(ea, B, H_q, H_kv, N, D, causal, seed, scale=None, dist="normal", mutate=None):
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N, D, seed, dist=dist)
    if mutate is not None:
        q, k, v = mutate(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o, l = _run(ea, q, k, v, causal, scale)
    O_ref, L_ref = oracle.attention_forward(workloads.to_float64(q), workloads.to_float64(k),
                                            workloads.to_float64(v), is_causal=causal,
                                            sm_scale=scale)
    return _check(o, l, O_ref, L_ref, what=f"B{B} Hq{H_q} Hkv{H_kv} N{N} D{D} c{int(causal)}")


# ------------------------------------------------------------ small workloads, full compare
SMALL = ["tiny_mha_n256_d64", "gqa4_b2_n1024", "mha_n512", "mqa_n512"]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("flip", [False, True], ids=["as_named", "causal_flipped"])
def test_small_workloads_full(ea, name, flip):
    w = workloads.WORKLOADS[name]
    causal = w.causal != flip
    _full_case(ea, w.B, w.H_q, w.H_kv, w.N, w.D, causal, w.seed)


def test_pages_shapes_listed():
    """The four shapes the first page checks are all among the parity cases."""
    with open(os.path.join(GOLDEN, "pages_numerical_shapes.json")) as f:
        shapes = json.load(f)["shapes"]
    have = {(w.B, w.H_q, w.H_kv, w.N, w.D) for w in workloads.WORKLOADS.values()}
    for s in shapes:
        assert (s["B"], s["H_q"], s["H_kv"], s["N"], s["D"]) in have


# ------------------------------------------------------------ full-size workloads, every row
LARGE = ["gqa8_n4096_causal", "gqa8_n4096_full", "gqa4_n8192_causal", "gqa4_n16384_causal",
         "gqa4_n32768_causal"]

_FULL = {}


def _full_init(q64, k64, v64, o, l):
    _FULL["t"] = (q64, k64, v64, o, l)


def _full_head(args):
    """Oracle for every row of head (b, h), compared with the GPU output."""
    from threadpoolctl import threadpool_limits
    b, h, causal, scale = args
    q64, k64, v64, o, l = _FULL["t"]
    with threadpool_limits(1):
        O_ref, L_ref = oracle.attention_rows(q64, k64, v64, b, h, np.arange(q64.shape[2]),
                                             is_causal=causal, sm_scale=scale)
    ob, lb = o[b, h].astype(np.float64), l[b, h].astype(np.float64)
    finite = bool(np.isfinite(ob).all() and np.isfinite(lb).all())
    err = np.abs(ob - O_ref)
    bad = int((err > O_ATOL + O_RTOL * np.abs(O_ref)).sum())
    return b, h, finite, bad, float(err.max()), float(np.abs(lb - L_ref).max())


@pytest.mark.parametrize("name", LARGE)
def test_large_workloads_full(ea, name):
    """Every output row of every head at the full workload sizes, in the
    launch configuration bench.py times, against the oracle.  The oracle runs
    one (batch, head) per task over a process pool (one worker per core, at
    most 16, one BLAS thread each; forked after the GPU run, the workers only
    run NumPy); about 10 s of CPU work at N = 32768."""
    import concurrent.futures as cf
    import multiprocessing
    w = workloads.WORKLOADS[name]
    print(f"[full] {name}", flush=True)
    q, k, v = workloads.workload_inputs(w)
    o, l = _run(ea, q, k, v, w.causal, w.sm_scale)
    q64, k64, v64 = (workloads.to_float64(t) for t in (q, k, v))
    o32, l32 = o.float().numpy(), l.numpy()
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    tasks = [(b, h, w.causal, w.sm_scale) for b in range(w.B) for h in range(w.H_q)]
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=multiprocessing.get_context("fork"),
                                initializer=_full_init, initargs=(q64, k64, v64, o32, l32)) as ex:
        results = list(ex.map(_full_head, tasks))
    worst_o = max(r[4] for r in results)
    worst_l = max(r[5] for r in results)
    print(f"[full] {name}: {len(results)} heads, max |dO| {worst_o:.3e}, max |dLSE| {worst_l:.3e}", flush=True)
    for b, h, finite, bad, eo, el in results:
        assert finite, f"{name} b{b} h{h}: non-finite output"
        assert bad == 0, f"{name} b{b} h{h}: {bad} O elements out of tolerance, max abs err {eo:.3e}"
        assert el <= LSE_ATOL, f"{name} b{b} h{h}: max LSE err {el:.3e}"


def test_large_d64_full(ea):
    """Every output row of causal GQA-4 N=16384 at D=64 against the oracle:
    the D=64 build of the eight-wave kernel at a grid long enough for the XCD
    work stealing (2048 workgroups).  Same process pool as above."""
    import concurrent.futures as cf
    import multiprocessing
    B, H_q, H_kv, N, D = 1, 32, 8, 16384, 64
    print(f"[full] d64 N={N}", flush=True)
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N, D, seed=964)
    scale = 1.0 / math.sqrt(D)
    o, l = _run(ea, q, k, v, True, scale)
    q64, k64, v64 = (workloads.to_float64(t) for t in (q, k, v))
    o32, l32 = o.float().numpy(), l.numpy()
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    tasks = [(b, h, True, scale) for b in range(B) for h in range(H_q)]
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=multiprocessing.get_context("fork"),
                                initializer=_full_init, initargs=(q64, k64, v64, o32, l32)) as ex:
        results = list(ex.map(_full_head, tasks))
    print(f"[full] d64: {len(results)} heads, max |dO| {max(r[4] for r in results):.3e}, "
          f"max |dLSE| {max(r[5] for r in results):.3e}", flush=True)
    for b, h, finite, bad, eo, el in results:
        assert finite, f"d64 b{b} h{h}: non-finite output"
        assert bad == 0, f"d64 b{b} h{h}: {bad} O elements out of tolerance, max abs err {eo:.3e}"
        assert el <= LSE_ATOL, f"d64 b{b} h{h}: max LSE err {el:.3e}"


def test_gqa8_n4096_some_heads_full(ea):
    """Two heads of different kv groups, every row, at the full GQA-8 shape."""
    w = workloads.WORKLOADS["gqa8_n4096_causal"]
    q, k, v = workloads.workload_inputs(w)
    q64, k64, v64 = (workloads.to_float64(t) for t in (q, k, v))
    for causal in (True, False):
        o, l = _run(ea, q, k, v, causal, w.sm_scale)
        for h in (5, 42):
            O_ref, L_ref = oracle.attention_rows(q64, k64, v64, 0, h, np.arange(w.N),
                                                 is_causal=causal, sm_scale=w.sm_scale)
            _check(o[0, h], l[0, h], O_ref, L_ref, what=f"gqa8 h{h} c{int(causal)}")


# ------------------------------------------------------------ edge cases
@pytest.mark.parametrize("N", [1, 2, 31, 33, 63, 65, 100, 129, 257, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(ea, N, D, causal):
    _full_case(ea, 1, 4, 2, N, D, causal, seed=7000 + N + D)


@pytest.mark.parametrize("H,D,causal", [(64, 128, False), (128, 64, True), (128, 128, True)])
def test_ragged_wide_grid(ea, H, D, causal):
    """N = 1000 over enough heads that the grid fills the 256 CUs (one round
    of eight-wave workgroups non-causal, two causal): the library takes the
    wide shape here, while the small cases above run the four-wave shape.
    Also through attn_fwd_splitkv with three forced key splits."""
    q, k, v = workloads.make_inputs(1, H, H, 1000, D, seed=7500 + H + D)
    scale = 1.0 / math.sqrt(D)
    O_ref, L_ref = oracle.attention_forward(workloads.to_float64(q), workloads.to_float64(k),
                                            workloads.to_float64(v), is_causal=causal, sm_scale=scale)
    o, l = _run(ea, q, k, v, causal, scale)
    _check(o, l, O_ref, L_ref, what=f"wide H{H} D{D} c{int(causal)}")
    dev = torch.device("cuda", 0)
    o, l = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), is_causal=causal, sm_scale=scale, n_splits=3)
    torch.cuda.synchronize()
    _check(o.cpu(), l.cpu(), O_ref, L_ref, what=f"wide split3 H{H} D{D} c{int(causal)}")


@pytest.mark.parametrize("D", [64, 128])
def test_wide_grid_last_tile_one_key(ea, D):
    """N = 65 over 256 kv heads, non-causal: one round of eight-wave
    workgroups, so the library takes the wide shape, whose last 64-key tile
    holds one key and 63 rows past the end.  Those rows come back from the
    tile's buffer range as zeros and must contribute nothing.  Also through
    attn_fwd_splitkv with three forced key splits."""
    q, k, v = workloads.make_inputs(1, 256, 256, 65, D, seed=7700 + D)
    scale = 1.0 / math.sqrt(D)
    O_ref, L_ref = oracle.attention_forward(workloads.to_float64(q), workloads.to_float64(k),
                                            workloads.to_float64(v), is_causal=False, sm_scale=scale)
    o, l = _run(ea, q, k, v, False, scale)
    _check(o, l, O_ref, L_ref, what=f"wide N65 D{D}")
    dev = torch.device("cuda", 0)
    o, l = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), is_causal=False, sm_scale=scale, n_splits=3)
    torch.cuda.synchronize()
    _check(o.cpu(), l.cpu(), O_ref, L_ref, what=f"wide N65 split3 D{D}")


@pytest.mark.parametrize("scale", [0.0, -0.088, 1.0])
def test_wide_grid_scale_values(ea, scale):
    """Zero, negative (Q negated on load) and large scales on a grid that
    takes the wide shape (GQA-2, 128 kv heads, N = 200, non-causal)."""
    q, k, v = workloads.make_inputs(1, 256, 128, 200, 128, seed=7800)
    O_ref, L_ref = oracle.attention_forward(workloads.to_float64(q), workloads.to_float64(k),
                                            workloads.to_float64(v), is_causal=False, sm_scale=scale)
    o, l = _run(ea, q, k, v, False, scale)
    _check(o, l, O_ref, L_ref, what=f"wide scale {scale}")


@pytest.mark.parametrize("H_q,H_kv", [(3, 3), (6, 2), (6, 1), (8, 4), (16, 2), (32, 2), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_head_groupings(ea, H_q, H_kv, causal):
    _full_case(ea, 2, H_q, H_kv, 96, 128, causal, seed=100 * H_q + H_kv)


@pytest.mark.parametrize("scale", [0.0, -0.088, 0.5, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_values(ea, scale, causal):
    """Zero (uniform weights), negative and large scales (peaked softmax)."""
    _full_case(ea, 1, 4, 1, 200, 128, causal, seed=31, scale=scale)


def test_identical_keys(ea):
    def same_keys(q, k, v):
        return q, k[:, :, :1].expand_as(k).contiguous(), v
    _full_case(ea, 1, 4, 2, 130, 128, True, seed=41, mutate=same_keys)


def test_growing_scores_force_rescaling(ea):
    """Key norms ramp from 0.2 to 12 along the sequence, so later scores climb
    far past the max the first tile sets and the tile-sum check (a sum of P
    above 2^24) takes its rescale branch on a small grid (the four-wave
    shape).  The premise is checked on the CPU: over 30 % of the rows past
    the first tile have a later score more than 24 (log2 units) above their
    first tile's max.  (A ramp to 3 climbs at most 17.4: P stays below 2^18
    and no tile rescales.)"""
    def ramp(q, k, v):
        g = torch.linspace(0.2, 12.0, k.shape[2]).view(1, 1, -1, 1)
        return q, (k.float() * g).to(torch.bfloat16), v
    q, k, v = workloads.make_inputs(1, 4, 4, 700, 128, 43)
    _, k, _ = ramp(q, k, v)
    s = np.einsum("bhnd,bhmd->bhnm", workloads.to_float64(q), workloads.to_float64(k)) / math.sqrt(128) / math.log(2.0)
    first = s[:, :, 64:, :64].max(axis=-1)
    later = s[:, :, 64:, 64:].max(axis=-1)
    assert np.mean(later - first > 24.0) > 0.3
    for causal in (False, True):
        _full_case(ea, 1, 4, 4, 700, 128, causal, seed=43, mutate=ramp)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_grid_forced_rescaling(ea, causal):
    """Key norms ramp from 0.1 to 25 along the sequence, so later scores
    climb far past the max the first tile sets: the tile-sum check (a sum of
    P above 2^24) must take its rescale branch.  The grid takes the wide
    shape (B=2, 128 kv heads, GQA-2, N = 200).  The premise is checked on the
    CPU: over 30 % of the rows past the first tile have a later score more
    than 24 (log2 units) above their first tile's max."""
    B, H_q, H_kv, N, D = 2, 256, 128, 200, 128
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N, D, seed=7900 + int(causal))
    ramp = torch.linspace(0.1, 25.0, N).view(1, 1, -1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    q64, k64, v64 = (workloads.to_float64(x) for x in (q, k, v))
    s = np.einsum("bhnd,bhmd->bhnm", q64, np.repeat(k64, H_q // H_kv, axis=1)) * scale / math.log(2.0)
    rows = np.arange(64, N)   # rows that see keys past the first tile (causal or not)
    first = s[:, :, rows, :64].max(axis=-1)
    later = np.where(np.arange(N)[None, None, None, :] <= rows[None, None, :, None], s[:, :, rows, :], -np.inf)[..., 64:].max(axis=-1)
    assert np.mean(later - first > 24.0) > 0.3
    O_ref, L_ref = oracle.attention_forward(q64, k64, v64, is_causal=causal, sm_scale=scale)
    o, l = _run(ea, q, k, v, causal, scale)
    _check(o, l, O_ref, L_ref, what=f"wide rescale c{int(causal)}")


@pytest.mark.parametrize("B,H_q,H_kv,N,causal", [
    (1, 32, 8, 4096, True),    # wide shape (16x16x32 MFMAs) for both runs
    (1, 32, 8, 4096, False),
    (2, 32, 8, 1024, True),    # mid shape (32x32x16 MFMAs) for both runs
    (1, 16, 1, 512, True),     # MQA: both runs split the keys, at different boundaries
])
def test_gqa_equals_own_mha_on_repeated_kv(ea, B, H_q, H_kv, N, causal):
    """Grouped-query attention equals this library's own multi-head run on K
    and V repeated to H_q heads (head h reads kv head h * H_kv / H_q; page
    "Triton Cuda Attention", section 变体改法, GQA).  Where both runs take the
    same kernel shape and no key split, every query sees the same K/V tiles
    in the same order with the same arithmetic, and i.i.d. N(0,1) inputs never
    take the rescale branch (a score 24 above the first tile's max), so the
    outputs are bit-identical; with key splits (MQA) the split boundaries
    differ and the two agree to the parity tolerance."""
    dev = torch.device("cuda", 0)
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N, 128, seed=9100 + N + H_kv)
    G = H_q // H_kv
    kr, vr = (x.repeat_interleave(G, dim=1).contiguous() for x in (k, v))
    o_g, l_g = _run(ea, q, k, v, causal, 1.0 / math.sqrt(128))
    o_m, l_m = _run(ea, q, kr, vr, causal, 1.0 / math.sqrt(128))
    splits_g = ea.attn_splitkv_num_splits(B, H_q, H_kv, N, N, 128, causal)
    splits_m = ea.attn_splitkv_num_splits(B, H_q, H_q, N, N, 128, causal)
    if splits_g == 1 and splits_m == 1:
        assert torch.equal(o_g.view(torch.int16), o_m.view(torch.int16)), "GQA and MHA outputs differ"
        assert torch.equal(l_g.view(torch.int32), l_m.view(torch.int32)), "GQA and MHA LSEs differ"
    else:
        assert splits_g > 1 and splits_m > 1
        o64 = o_m.to(torch.float64).numpy()
        _check(o_g, l_g, o64, l_m.to(torch.float64).numpy(), what="GQA vs own MHA")
    O_ref, L_ref = oracle.attention_forward(workloads.to_float64(q), workloads.to_float64(k),
                                            workloads.to_float64(v), is_causal=causal,
                                            sm_scale=1.0 / math.sqrt(128))
    _check(o_g, l_g, O_ref, L_ref, what="GQA vs oracle")


@pytest.mark.parametrize("scale", [1e3, 1e6, -1e6])
def test_large_scales_peaked_softmax(ea, scale):
    """Scales far above 1/sqrt(D): each row's softmax is one-hot on its largest
    score (the second largest is at least 1e-3 below it here, checked on the
    CPU, so the weight of any other key is below e^-1), O is that key's V row
    and the LSE is the largest scaled score, of order 1e7 at scale 1e6.  The
    LSE bound is relative there: the fp32 score carries the rounding of its
    128-term dot product, of order 2^-24 times the sum of |q_d k_d| (a few
    times the score itself for N(0,1) data), and the scale multiplies it, so
    the bound is 2^-20 of |LSE| on top of 1e-3.  Within the documented range
    (scaled scores below 2^31 in log2 units) the kernel's exponent of the
    largest score is the rounding error of that score times the scale, which
    stays small."""
    B, H_q, H_kv, N, D = 1, 4, 2, 300, 128
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N, D, seed=9300)
    q64, k64, v64 = (workloads.to_float64(x) for x in (q, k, v))
    for causal in (False, True):
        s = scale * np.einsum("bhnd,bhmd->bhnm", q64, np.repeat(k64, 2, axis=1))
        if causal:
            s = np.where(np.arange(N)[None, None, None, :] > np.arange(N)[None, None, :, None], -np.inf, s)
        srt = np.sort(s, axis=-1)
        gap = (srt[..., -1] - srt[..., -2])[:, :, 1:]   # row 0 of causal sees one key
        assert gap.min() > 1.0
        assert np.abs(srt[..., -1]).max() / math.log(2.0) < 2.0 ** 31
        O_ref, L_ref = oracle.attention_forward(q64, k64, v64, is_causal=causal, sm_scale=scale)
        o, l = _run(ea, q, k, v, causal, scale)
        o64, l64 = o.to(torch.float64).numpy(), l.to(torch.float64).numpy()
        assert np.all(np.isfinite(o64)) and np.all(np.isfinite(l64))
        assert np.all(np.abs(o64 - O_ref) <= O_ATOL + O_RTOL * np.abs(O_ref)), f"O at scale {scale}"
        rel = float(np.max(np.abs(l64 - L_ref) / np.maximum(np.abs(L_ref), 1.0)))
        assert np.all(np.abs(l64 - L_ref) <= LSE_ATOL + 2.0 ** -20 * np.abs(L_ref)), \
            f"LSE at scale {scale}: max relative error {rel:.3e}"


def test_uniform_inputs_d64(ea):
    _full_case(ea, 2, 8, 2, 300, 64, True, seed=44, dist="uniform")


# ------------------------------------------------------------ hygiene
def test_empty_inputs(ea):
    dev = torch.device("cuda", 0)
    q = torch.empty((0, 4, 16, 128), dtype=torch.bfloat16, device=dev)
    k = torch.empty((0, 2, 16, 128), dtype=torch.bfloat16, device=dev)
    out, lse = ea.fwd(q, k, k, is_causal=True)
    assert out.shape == q.shape and lse.shape == (0, 4, 16)
    q = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device=dev)
    k = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device=dev)
    out, lse = ea.fwd(q, k, k)
    assert out.numel() == 0


def test_deterministic_and_no_overrun(ea):
    """Two runs agree bit for bit; bytes just past out and lse stay untouched."""
    dev = torch.device("cuda", 0)
    q, k, v = workloads.make_inputs(1, 8, 2, 333, 128, seed=51)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    n_o, n_l = q.numel(), q.numel() // 128
    res = []
    for _ in range(2):
        ob = torch.full((n_o + 4096,), 7.0, dtype=torch.bfloat16, device=dev)
        lb = torch.full((n_l + 1024,), 7.0, dtype=torch.float32, device=dev)
        out = ob[:n_o].view(q.shape)
        lse = lb[:n_l].view(1, 8, 333)
        ea.attn_fwd(qd, kd, vd, out, lse, is_causal=True)
        torch.cuda.synchronize()
        assert torch.all(ob[n_o:] == 7.0) and torch.all(lb[n_l:] == 7.0), "overrun"
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1], res[1][1])


def test_side_stream(ea):
    dev = torch.device("cuda", 0)
    q, k, v = workloads.make_inputs(1, 4, 4, 256, 128, seed=52)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ref_o, ref_l = ea.fwd(qd, kd, vd, is_causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, l = ea.fwd(qd, kd, vd, is_causal=True)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(l, ref_l)


def test_concurrent_host_threads(ea):
    """Two host threads enqueue forwards (single pass and key splits) on
    their own streams at the same time; every result equals, bit for bit,
    the same call made alone: no result depends on another call."""
    import threading
    dev = torch.device("cuda", 0)
    cases = []
    for i, (H_q, H_kv, N, n_splits) in enumerate([(8, 2, 700, 1), (4, 4, 513, 3)]):
        q, k, v = workloads.make_inputs(1, H_q, H_kv, N, 128, seed=60 + i)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        ref = ea.fwd_splitkv(qd, kd, vd, is_causal=True, n_splits=n_splits)
        cases.append((qd, kd, vd, n_splits, ref))
    torch.cuda.synchronize()
    results = [[None] * 10 for _ in cases]
    errors = []

    def worker(j):
        try:
            qd, kd, vd, n_splits, _ = cases[j]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(10):
                    results[j][it] = ea.fwd_splitkv(qd, kd, vd, is_causal=True, n_splits=n_splits)
            s.synchronize()
        except Exception as exc:  # reported below, in the test's thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (_, _, _, _, (ro, rl)), res in zip(cases, results):
        for o, l in res:
            assert torch.equal(o.view(torch.int16), ro.view(torch.int16)) and torch.equal(l, rl)


@pytest.mark.parametrize("D", [128, 64])
def test_work_stealing_schedule(ea, D):
    """A long single pass (causal GQA-4, N = 16384, D = 128 and 64: eight
    rounds of the device) lets the XCDs claim work through per-stream counters; captured
    into a graph it runs the static work order.  Every schedule gives the
    same bits: repeated calls on one stream (each launch must leave its
    counters at zero for the next), two streams running at once (separate
    counters), two host threads on their own streams, the per-thread default
    stream and graph replays interleaved with eager calls (both in the static
    order)."""
    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS["gqa4_n16384_causal"]
    print(f"[steal] {w.name} D={D}", flush=True)
    if D == 128:
        q, k, v = (x.to(dev) for x in workloads.workload_inputs(w))
    else:
        w = dataclasses.replace(w, D=64)
        q, k, v = (x.to(dev) for x in workloads.make_inputs(w.B, w.H_q, w.H_kv, w.N, 64, seed=w.seed + 64))

    def bufs():
        return (torch.full(w.q_shape(), float("nan"), dtype=torch.bfloat16, device=dev),
                torch.full((w.B, w.H_q, w.Nq), float("nan"), dtype=torch.float32, device=dev))

    def same(a, b):
        return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])

    ref = bufs()
    ea.attn_fwd(q, k, v, *ref, is_causal=True, sm_scale=w.sm_scale)
    for _ in range(3):
        o = bufs()
        ea.attn_fwd(q, k, v, *o, is_causal=True, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert same(o, ref), "repeated call on one stream differs"
    assert bool(torch.isfinite(ref[0]).all()) and bool(torch.isfinite(ref[1]).all())

    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [bufs() for _ in streams]
    torch.cuda.synchronize()
    for it in range(3):
        for s, o in zip(streams, outs):
            with torch.cuda.stream(s):
                ea.attn_fwd(q, k, v, *o, is_causal=True, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        for o in outs:
            assert same(o, ref), f"concurrent streams, round {it}: result differs"

    # two host threads, each on its own stream, claim counter slots at once
    import threading
    t_outs = [[bufs() for _ in range(2)] for _ in range(2)]
    errors = []
    torch.cuda.synchronize()

    def worker(j):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for o in t_outs[j]:
                    ea.attn_fwd(q, k, v, *o, is_causal=True, sm_scale=w.sm_scale)
            st.synchronize()
        except Exception as exc:  # reported below, in the test's thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j in range(2):
        for o in t_outs[j]:
            assert same(o, ref), f"host thread {j}: result differs"

    # hipStreamPerThread (handle 2) names a different stream in every thread:
    # the static order
    o = bufs()
    torch.cuda.synchronize()
    ea.attn_fwd(q, k, v, *o, is_causal=True, sm_scale=w.sm_scale, stream=2)
    torch.cuda.synchronize()
    assert same(o, ref), "per-thread default stream differs"

    g_out = bufs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ea.attn_fwd(q, k, v, *g_out, is_causal=True, sm_scale=w.sm_scale)
    for it in range(3):
        g_out[0].fill_(float("nan"))
        g_out[1].fill_(float("nan"))
        graph.replay()
        o = bufs()
        ea.attn_fwd(q, k, v, *o, is_causal=True, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert same(g_out, ref), f"graph replay {it} (static order) differs"
        assert same(o, ref), f"eager call after replay {it} differs"


def test_status_error_raises(ea):
    dev = torch.device("cuda", 0)
    q = torch.zeros((1, 4, 16, 96), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ea.AttnError) as e:
        ea.fwd(q, q, q)
    assert e.value.status == 3
    assert e.value.call == "attn_fwd" and "attn_fwd failed with status 3" in str(e.value)
