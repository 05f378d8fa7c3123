"""GPU parity of the attention backward (dQ, dK, dV) against the float64 CPU
oracle.

Inputs are seeded bf16 Q, K, V and dO.  Unless a case says otherwise, the
forward output O (rounded to bf16) and the LSE (fp32) handed to the backward
are the oracle's, so that the backward is checked on its own; the chained
cases feed it this library's own forward instead.  The forward output is an
operand of the backward (Dl = rowsum(dO * out)), so the oracle is given the
same bf16 output the kernel receives.

Tolerance (the pages give none for gradients; the forward's bf16 allclose of
page "Attention Kernel 实现与正确性验证", section 1.3, made scale-free):
element-wise |g - r| <= 2e-2 s + 2e-2 |r|, where s is the larger of the root
mean square of the reference row (the D values of one query row of dQ, or of
one key of dK, dV) and of the whole reference tensor, at least 1e-4 (fp32
round-off where the reference is exactly zero); nothing non-finite.  P
and dS are rounded to bf16 before their products (relative 2^-9 each), so the
error of a gradient row scales with that row's own magnitude: early causal
rows, which see few keys, have gradients ten times the tensor's typical size
(a CPU emulation of the rounding reproduces their errors).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

G_ATOL = 2e-2   # times rms of the reference tensor
G_RTOL = 2e-2
G_FLOOR = 1e-4  # least row scale: fp32 round-off of gradients that are exactly zero


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_02_amd as m
    m.load_library()
    return m


def _dev():
    return torch.device("cuda", 0)


def _inputs(B, H_q, H_kv, N_q, N_kv, D, seed):
    q, k, v = workloads.make_inputs(B, H_q, H_kv, N_q, D, seed, N_kv=N_kv)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    dO = torch.randn((B, H_q, N_q, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, dO


def _check(name, got, ref, what):
    g = got.to(torch.float64).numpy() if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    s = np.maximum(np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)), max(rms, G_FLOOR))
    err = np.abs(g - ref)
    bad = err > G_ATOL * s + G_RTOL * np.abs(ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} {name} elements out of tolerance; "
                           f"max err {err.max():.3e}, rms(ref) {rms:.3e}")


def _run_bwd(ea, q, k, v, o, dO, lse, causal, scale, poison=True, n_splits=0):
    dev = _dev()
    t = [x.to(dev) for x in (q, k, v, o, dO)]
    lsed = lse.to(dev)
    dq = torch.empty_like(t[0])
    dk = torch.empty_like(t[1])
    dv = torch.empty_like(t[2])
    if poison:
        for x in (dq, dk, dv):
            x.fill_(float("nan"))
    B, H_q, N_q, D = q.shape
    H_kv, N_kv = k.shape[1], k.shape[2]
    ns = n_splits if n_splits > 0 else max(ea.attn_bwd_num_splits(B, H_q, H_kv, N_q, N_kv, D, causal), 1)
    nbytes = ea.attn_bwd_workspace_size(B, H_q, H_kv, N_q, N_kv, D, causal, ns)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=dev)
    ea.attn_bwd(t[0], t[1], t[2], t[3], t[4], lsed, dq, dk, dv, is_causal=causal, sm_scale=scale,
                n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _oracle_fwd_outputs(q64, k64, v64, causal, scale):
    O, L = oracle.attention_forward(q64, k64, v64, is_causal=causal, sm_scale=scale)
    return torch.from_numpy(O).to(torch.bfloat16), torch.from_numpy(L).to(torch.float32)


def _case(ea, B, H_q, H_kv, N_q, N_kv, D, causal, seed, scale=None, chained=False, mutate=None,
          n_splits=0):
    q, k, v, dO = _inputs(B, H_q, H_kv, N_q, N_kv, D, seed)
    if mutate is not None:
        q, k, v, dO = mutate(q, k, v, dO)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q64, k64, v64, d64 = (workloads.to_float64(x) for x in (q, k, v, dO))
    if chained:
        dev = _dev()
        o, lse = ea.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), is_causal=causal,
                                sm_scale=scale, n_splits=1)
        o, lse = o.cpu(), lse.cpu()
    else:
        o, lse = _oracle_fwd_outputs(q64, k64, v64, causal, scale)
    dq, dk, dv = _run_bwd(ea, q, k, v, o, dO, lse, causal, scale, n_splits=n_splits)
    rq, rk, rv = oracle.attention_backward(q64, k64, v64, d64, is_causal=causal, sm_scale=scale,
                                           out=workloads.to_float64(o))
    what = f"B{B} Hq{H_q} Hkv{H_kv} Nq{N_q} Nkv{N_kv} D{D} c{int(causal)} s{scale:.3g} ns{n_splits}"
    _check("dQ", dq, rq, what)
    _check("dK", dk, rk, what)
    _check("dV", dv, rv, what)


@pytest.mark.parametrize("shape", [
    (1, 4, 4, 128, 128, 128), (2, 8, 2, 300, 300, 128), (1, 4, 1, 257, 257, 64),
    (1, 6, 2, 100, 100, 128), (1, 8, 8, 64, 64, 64), (1, 3, 3, 200, 200, 128),
], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small(ea, shape, causal):
    _case(ea, *shape, causal, seed=12000 + sum(shape))


@pytest.mark.parametrize("N", [1, 2, 31, 33, 65, 129, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged(ea, N, D, causal):
    _case(ea, 1, 4, 2, N, N, D, causal, seed=12100 + N + D)


@pytest.mark.parametrize("N_q,N_kv", [(1, 777), (64, 500), (100, 1000), (5, 33), (300, 100)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_rectangular(ea, N_q, N_kv, causal):
    if causal and N_q > N_kv:
        pytest.skip("causal needs N_q <= N_kv")
    _case(ea, 1, 8, 2, N_q, N_kv, 128, causal, seed=12200 + N_q + N_kv)


@pytest.mark.parametrize("B,H_q,H_kv,N_q,N_kv,D,causal", [
    (2, 128, 128, 100, 100, 128, False),   # 256 dQ workgroups: one round of eight waves
    (2, 256, 128, 90, 90, 64, False),      # GQA-2, two pairs per head row
    (2, 256, 256, 100, 100, 128, True),    # causal: 512 workgroups, two rounds
    (2, 128, 128, 60, 300, 128, True),     # causal chunk, N_q < N_kv / 2
])
def test_backward_eight_wave_dq(ea, B, H_q, H_kv, N_q, N_kv, D, causal):
    """Grids large enough for the eight-wave dQ kernel (16x16x32 MFMAs, two
    pairs per lane) at sizes the oracle checks element by element; the
    smaller cases above run the four-wave kernel."""
    _case(ea, B, H_q, H_kv, N_q, N_kv, D, causal, seed=8100 + H_q + N_q)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_backward_scale_values(ea, scale):
    _case(ea, 1, 4, 2, 150, 150, 128, True, seed=12300, scale=scale)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("shape", [
    (1, 16, 1, 512, 512, 128, True), (1, 6, 2, 100, 100, 64, False), (2, 4, 1, 70, 300, 128, True),
    (1, 3, 1, 1, 129, 128, True), (1, 8, 2, 200, 200, 128, False),
], ids=lambda s: "x".join(map(str, s)))
def test_backward_row_range_splits(ea, shape, n_splits):
    """dK/dV with a key block's (head, row tile) sequence cut into n_splits
    ranges (more ranges than tiles leaves some empty) and summed in order."""
    B, H_q, H_kv, N_q, N_kv, D, causal = shape
    _case(ea, B, H_q, H_kv, N_q, N_kv, D, causal, seed=12700 + N_q + n_splits, n_splits=n_splits)


def test_backward_mqa_workload(ea):
    """Causal MQA N=512 (16 query heads on one kv head) with the library's split."""
    w = workloads.WORKLOADS["mqa_n512"]
    assert ea.attn_bwd_num_splits(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.causal) > 1
    _case(ea, w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.causal, seed=w.seed)


def test_backward_workload_gqa4_b2_n1024(ea):
    w = workloads.WORKLOADS["gqa4_b2_n1024"]
    _case(ea, w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.causal, seed=w.seed)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_chained_with_forward(ea, causal):
    """This library's forward output and LSE feed its backward."""
    _case(ea, 2, 8, 2, 333, 333, 128, causal, seed=12400, chained=True)
    _case(ea, 1, 8, 2, 40, 600, 64, causal, seed=12401, chained=True)


def test_backward_identical_keys(ea):
    """All keys equal: the exact dQ is zero, a total cancellation of terms
    whose bf16 rounding does not cancel.  dK and dV follow the usual rule; dQ
    is bounded with the row scale s taken from the reference dQ of the same Q
    and dO with the original keys, the typical size of those terms."""
    B, H_q, H_kv, N, D, seed = 1, 4, 2, 130, 128, 12500
    q, k0, v, dO = _inputs(B, H_q, H_kv, N, N, D, seed)
    k = k0[:, :, :1].expand_as(k0).contiguous()
    sc = 1.0 / math.sqrt(D)
    q64, k64, v64, d64 = (workloads.to_float64(x) for x in (q, k, v, dO))
    o, lse = _oracle_fwd_outputs(q64, k64, v64, True, sc)
    o64 = workloads.to_float64(o)
    dq, dk, dv = _run_bwd(ea, q, k, v, o, dO, lse, True, sc)
    rq, rk, rv = oracle.attention_backward(q64, k64, v64, d64, is_causal=True, sm_scale=sc, out=o64)
    _check("dK", dk, rk, "identical keys")
    _check("dV", dv, rv, "identical keys")
    rq0, _, _ = oracle.attention_backward(q64, workloads.to_float64(k0), v64, d64, is_causal=True,
                                          sm_scale=sc, out=o64)
    rms0 = float(np.sqrt(np.mean(rq0 * rq0)))
    s_row = np.maximum(np.sqrt(np.mean(rq0 * rq0, axis=-1, keepdims=True)), rms0)
    err = np.abs(dq.to(torch.float64).numpy() - rq)
    assert np.all(err <= G_ATOL * s_row), float((err / s_row).max())


def test_backward_large_sampled(ea):
    """Causal GQA-8 N=4096 at full size: dQ of sampled rows, dK/dV of sampled
    keys of two kv heads, against the oracle's row and key entry points."""
    w = workloads.WORKLOADS["gqa8_n4096_causal"]
    q, k, v, dO = _inputs(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.seed)
    dev = _dev()
    o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), is_causal=True)
    dq, dk, dv = _run_bwd(ea, q, k, v, o.cpu(), dO, lse.cpu(), True, w.sm_scale)
    q64, k64, v64, d64, o64 = (workloads.to_float64(x) for x in (q, k, v, dO, o.cpu()))
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 2047, 4094, 4095], rng.choice(w.N, 6, replace=False)]))
    for h in (0, 37):
        r = oracle.backward_rows(q64, k64, v64, d64, 0, h, rows, is_causal=True, sm_scale=w.sm_scale,
                                 out=o64)
        _check("dQ", dq[0, h, rows], r, f"gqa8 dQ h{h}")
    keys = np.unique(np.concatenate([[0, 1, 127, 128, 4095], rng.choice(w.N, 5, replace=False)]))
    for g in (0, 5):
        rk, rv = oracle.backward_keys(q64, k64, v64, d64, 0, g, keys, is_causal=True,
                                      sm_scale=w.sm_scale, out=o64)
        _check("dK", dk[0, g, keys], rk, f"gqa8 dK g{g}")
        _check("dV", dv[0, g, keys], rv, f"gqa8 dV g{g}")


def test_backward_no_query_rows(ea):
    dev = _dev()
    q = torch.empty((1, 4, 0, 128), dtype=torch.bfloat16, device=dev)
    k = torch.randn((1, 2, 50, 128), device=dev).to(torch.bfloat16)
    lse = torch.empty((1, 4, 0), dtype=torch.float32, device=dev)
    dq, dk, dv = ea.bwd(q, k, k, q, q, lse, is_causal=True)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_deterministic_and_no_overrun(ea):
    dev = _dev()
    q, k, v, dO = (x.to(dev) for x in _inputs(1, 8, 2, 333, 333, 128, 12600))
    o, lse = ea.fwd(q, k, v, is_causal=True)
    res = []
    for _ in range(2):
        bufs = [torch.full((x.numel() + 4096,), 7.0, dtype=torch.bfloat16, device=dev) for x in (q, k, v)]
        dq, dk, dv = (b[:x.numel()].view(x.shape) for b, x in zip(bufs, (q, k, v)))
        need = ea.attn_bwd_workspace_size(1, 8, 2, 333, 333, 128, True, 5)
        wb = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device=dev)
        ea.attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, is_causal=True, n_splits=5, workspace=wb[:need])
        torch.cuda.synchronize()
        for b, x in zip(bufs, (q, k, v)):
            assert torch.all(b[x.numel():] == 7.0), "overrun"
        assert torch.all(wb[need:] == 0x5A), "workspace overrun"
        res.append([t.clone() for t in (dq, dk, dv)])
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


_BW = {}


def _bw_init(q64, k64, v64, d64, o64):
    _BW["t"] = (q64, k64, v64, d64, o64)


def _bw_keys_task(args):
    """dK, dV of the sampled keys of kv head g, summed over one block of query
    rows of every head of the group (the parent sums the blocks)."""
    from threadpoolctl import threadpool_limits
    g, keys, rows, scale = args
    q64, k64, v64, d64, o64 = _BW["t"]
    with threadpool_limits(1):
        return g, oracle.backward_keys(q64, k64, v64, d64, 0, g, keys, is_causal=True, sm_scale=scale,
                                       out=o64, rows=rows)


def _bw_rows_task(args):
    from threadpoolctl import threadpool_limits
    h, rows, scale = args
    q64, k64, v64, d64, o64 = _BW["t"]
    with threadpool_limits(1):
        return h, oracle.backward_rows(q64, k64, v64, d64, 0, h, rows, is_causal=True, sm_scale=scale,
                                       out=o64)


@pytest.mark.parametrize("name", ["gqa4_n8192_causal", "gqa4_n32768_causal"])
def test_backward_timed_workloads_sampled(ea, name):
    """The backward at the shapes its throughput is quoted on (causal GQA-4,
    B=1, H_q=32, H_kv=8, D=128), in the library's default launch (the split
    count attn_bwd_num_splits picks), fed this library's own forward output
    and LSE.  dQ of sampled rows (first and last row tiles, both sides of
    64- and 128-row boundaries, random rows) of every head of two kv groups,
    and dK/dV of sampled keys (0, 127, 128, N-1, random) of the same two kv
    groups summed over every query row, against the oracle's row and key
    entry points.  The key sums run over a process pool in blocks of 512 rows
    (about 200 CPU-seconds at N = 32768)."""
    import concurrent.futures as cf
    import multiprocessing
    import os
    w = workloads.WORKLOADS[name]
    print(f"[bwd-timed] {name}", flush=True)
    q, k, v, dO = _inputs(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.seed)
    dev = _dev()
    o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), is_causal=True)
    o, lse = o.cpu(), lse.cpu()
    dq, dk, dv = _run_bwd(ea, q, k, v, o, dO, lse, True, w.sm_scale)
    print(f"[bwd-timed] {name}: GPU done, oracle next", flush=True)
    q64, k64, v64, d64, o64 = (workloads.to_float64(x) for x in (q, k, v, dO, o))
    N, G = w.N, w.H_q // w.H_kv
    rng = np.random.default_rng(w.seed + 1)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N // 2 - 1, N // 2, N - 129, N - 128,
                                      N - 65, N - 64, N - 2, N - 1], rng.choice(N, 6, replace=False)]))
    keys = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 2, N - 1], rng.choice(N, 5, replace=False)]))
    groups = (0, w.H_kv - 1)
    heads = [g * G + j for g in groups for j in range(G)]
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    key_tasks = [(g, keys, np.arange(r0, min(r0 + 512, N)), w.sm_scale)
                 for g in groups for r0 in range(0, N, 512)]
    rk = {g: np.zeros((keys.size, w.D)) for g in groups}
    rv = {g: np.zeros((keys.size, w.D)) for g in groups}
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=multiprocessing.get_context("fork"),
                                initializer=_bw_init, initargs=(q64, k64, v64, d64, o64)) as ex:
        row_res = list(ex.map(_bw_rows_task, [(h, rows, w.sm_scale) for h in heads]))
        for g, (a, b_) in ex.map(_bw_keys_task, key_tasks):
            rk[g] += a
            rv[g] += b_
    for h, r in row_res:
        _check("dQ", dq[0, h, rows], r, f"{name} dQ h{h}")
    for g in groups:
        _check("dK", dk[0, g, keys], rk[g], f"{name} dK g{g}")
        _check("dV", dv[0, g, keys], rv[g], f"{name} dV g{g}")
    print(f"[bwd-timed] {name}: {len(heads)} heads x {rows.size} rows, {len(groups)} groups x "
          f"{keys.size} keys pass", flush=True)


@pytest.mark.parametrize("D", [128, 64])
def test_backward_stealing_schedule(ea, D):
    """At causal GQA-4 N=32768 (D=128 and 64) both backward kernels have grids of at least
    eight rounds of the device, so their workgroups claim work between the
    XCDs through the stream's counters; captured into a graph the same call
    runs the static order.  dQ, dK and dV agree bit for bit across repeated
    eager calls (each launch must leave the counters at zero) and graph
    replays interleaved with eager calls."""
    w = workloads.WORKLOADS["gqa4_n32768_causal"]
    if D != w.D:
        w = dataclasses.replace(w, D=D, seed=w.seed + D)
    print(f"[bwd-steal] {w.name} D={D}", flush=True)
    dev = _dev()
    q, k, v, dO = (x.to(dev) for x in _inputs(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, w.seed))
    o, lse = ea.fwd(q, k, v, is_causal=True)
    ns = ea.attn_bwd_num_splits(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, True)
    ws = torch.empty(ea.attn_bwd_workspace_size(w.B, w.H_q, w.H_kv, w.N, w.N, w.D, True, ns),
                     dtype=torch.uint8, device=dev)

    def grads():
        return tuple(torch.full_like(x, float("nan")) for x in (q, k, v))

    def run(g):
        ea.attn_bwd(q, k, v, o, dO, lse, *g, is_causal=True, sm_scale=w.sm_scale, n_splits=ns, workspace=ws)

    def same(a, b):
        return all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))

    ref = grads()
    run(ref)
    torch.cuda.synchronize()
    for it in range(2):
        g = grads()
        run(g)
        torch.cuda.synchronize()
        assert same(g, ref), f"repeated eager call {it} differs"
    g_out = grads()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g_out)
    for it in range(2):
        for x in g_out:
            x.fill_(float("nan"))
        graph.replay()
        g = grads()
        run(g)
        torch.cuda.synchronize()
        assert same(g_out, ref), f"graph replay {it} (static order) differs"
        assert same(g, ref), f"eager call after replay {it} differs"


@pytest.mark.parametrize("N_q,N_kv,D,causal", [(200, 200, 128, True), (200, 200, 64, False), (96, 300, 128, True)])
def test_autograd_wrapper(ea, N_q, N_kv, D, causal):
    """ea.attention as a torch.autograd.Function: its output and the q, k, v
    gradients that autograd returns are bit for bit those of the direct
    entry points (forward, then attn_bwd on the saved O and LSE), and agree
    with the oracle's gradients of the same loss within the backward
    tolerance."""
    q, k, v, dO = _inputs(1, 4, 2, N_q, N_kv, D, seed=4400 + N_q + D)
    dev = _dev()
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    out = ea.attention(qd, kd, vd, is_causal=causal)
    out.backward(dO.to(dev))
    torch.cuda.synchronize()
    qp, kp, vp = q.to(dev), k.to(dev), v.to(dev)
    if N_q == N_kv:
        o_ref, l_ref = ea.fwd(qp, kp, vp, is_causal=causal)
    else:
        o_ref, l_ref = ea.fwd_splitkv(qp, kp, vp, is_causal=causal)
    dq, dk, dv = ea.bwd(qp, kp, vp, o_ref, dO.to(dev), l_ref, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out.detach().view(torch.int16), o_ref.view(torch.int16))
    for name, got, ref in (("dQ", qd.grad, dq), ("dK", kd.grad, dk), ("dV", vd.grad, dv)):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name} differs from attn_bwd"
    q64, k64, v64, d64 = (workloads.to_float64(x) for x in (q, k, v, dO))
    rq, rk, rv = oracle.attention_backward(q64, k64, v64, d64, is_causal=causal, sm_scale=scale,
                                           out=workloads.to_float64(o_ref.cpu()))
    _check("dQ", qd.grad.cpu(), rq, f"autograd {N_q}x{N_kv} D{D}")
    _check("dK", kd.grad.cpu(), rk, f"autograd {N_q}x{N_kv} D{D}")
    _check("dV", vd.grad.cpu(), rv, f"autograd {N_q}x{N_kv} D{D}")


def _draw_backward_cases(seed: int = 20261202, n: int = 12):
    """Seeded random backward problems in four groups, so that every launch
    shape runs: many kv heads with short rows (the eight-wave dQ kernel);
    small square grids with a drawn row-range split count (the four-wave dQ
    kernel, partial dK/dV sums); causal chunks with N_q < N_kv (bottom-right
    mask); and square grids fed this library's own forward (chained)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = i % 4
        D = int(rng.choice([64, 128]))
        n_splits, chained = 0, False
        if kind == 0:
            B, H_kv, G = 2, 128, int(rng.choice([1, 2]))
            N_q = int(rng.integers(65, 256 // G + 1))
            N_kv = N_q if rng.random() < 0.5 else int(rng.integers(N_q, 400))
            causal = bool(rng.random() < 0.3)
        elif kind == 1:
            B, H_kv, G = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 4, 8]))
            N_q = N_kv = int(rng.integers(2, 600))
            causal = bool(rng.random() < 0.5)
            n_splits = int(rng.choice([0, 1, 2, 3, 5]))
        elif kind == 2:
            B, H_kv, G = 1, int(rng.choice([2, 8])), int(rng.choice([1, 4]))
            N_q = int(rng.integers(1, 300))
            N_kv = int(rng.integers(N_q, 900))
            causal = True
        else:
            B, H_kv, G = int(rng.integers(1, 3)), int(rng.choice([1, 4, 8])), int(rng.choice([1, 2, 4]))
            N_q = N_kv = int(rng.integers(2, 500))
            causal = bool(rng.random() < 0.5)
            chained = True
        cases.append((B, H_kv * G, H_kv, N_q, N_kv, D, causal, n_splits, chained, 9500 + i))
    return cases


@pytest.mark.parametrize("B,H_q,H_kv,N_q,N_kv,D,causal,n_splits,chained,seed", _draw_backward_cases())
def test_backward_random_shapes(ea, B, H_q, H_kv, N_q, N_kv, D, causal, n_splits, chained, seed):
    """dQ, dK and dV of every element against the oracle on a seeded random
    shape (the draw is fixed, so the cases are the same on every run)."""
    _case(ea, B, H_q, H_kv, N_q, N_kv, D, causal, seed=seed, chained=chained, n_splits=n_splits)
