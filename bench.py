#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (every query row of
every head), inputs already resident in HBM.  Default workload: long-context
causal GQA-4, B=1, H_q=32, H_kv=8, N=32768, D=128, bf16 i.i.d. N(0,1).

Prints ONE JSON line with the throughput in attention TFLOP/s
(4*B*H_q*N^2*D, halved for causal), the roofline of the kernel (MFMA-bound:
achieved TFLOP/s per launch from HIP events on the launch stream, against the
2.5 PFLOP/s dense bf16 peak, and against the same MFMA rate at the shader
clock measured during the kernel when a counter summary for the current
sources is committed), a CPU baseline (the float64 oracle on a bounded
sample of the same workload, on the host's cores) and a parity check of
every row of the timed output against the oracle.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--sweep]
    python bench.py --backward-sweep | --mla-sweep      (tables to stderr)
    python bench.py --backward --workload NAME | --mla NAME [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
MFMA_FLOP_PER_CLK = 256 * 4096  # dense bf16 MFMA, whole chip (2.5 PFLOP/s at 2.4 GHz)
METRIC = "attention fwd TFLOPS and % of MI355X bf16 MFMA peak (GQA causal, N=1K–32K)"
CSRC = os.path.join(ROOT, "exact_attention_02_amd", "csrc")
# Sources whose hash ties a committed profile to the kernels it measured; the
# build script is part of each list because its per-source flags change the
# binaries too.
BUILD_SCRIPT = os.path.join(ROOT, "exact_attention_02_amd", "build.py")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("attn_fwd_kernel.hpp", "attn_abi.hip")] + [BUILD_SCRIPT]
BWD_SOURCES = [os.path.join(CSRC, f) for f in ("attn_bwd_kernel.hpp", "attn_bwd.hip")] + [BUILD_SCRIPT]
# the latent core's kernels: attn_mla_kernel and the forward header's merge
MLA_SOURCES = [os.path.join(CSRC, f) for f in ("attn_mla_kernel.hpp", "attn_mla.hip", "attn_fwd_kernel.hpp")] + [BUILD_SCRIPT]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in (sources or KERNEL_SOURCES):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_profile(name: str, key: str, sources=None):
    """A figure (`key: value`) from a committed rocprofv3 summary under
    profiles/, or None when the file is missing or its kernel-source hash
    differs from the current sources (a figure of other kernels)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_v = re.search(re.escape(key) + r":\s*([0-9.eE+-]+)", txt)
    if not m_hash or not m_v or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_v.group(1))


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary (or None)."""
    return read_profile(f"attn_fwd_{workload}_hbm_traffic.md", "hbm_bytes_per_launch")


def read_clock(workload: str):
    """Shader clock (GHz) during the kernel from the committed counter summary
    (GRBM_COUNT over the dispatch), or None."""
    return read_profile(f"attn_fwd_{workload}_counters.md", "shader_clock_ghz")


def read_mfma_busy(workload: str):
    """Fraction of SIMD cycles with the MFMA pipe busy during the kernel, from
    the same summary (SQ_VALU_MFMA_BUSY_CYCLES), or None."""
    return read_profile(f"attn_fwd_{workload}_counters.md", "mfma_busy_frac")


# ---------------------------------------------------------------- CPU baseline
def _oracle_unit(args):
    from threadpoolctl import threadpool_limits
    import oracle
    q, k, v, b, h, rows, causal, scale = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, b, h, rows, is_causal=causal, sm_scale=scale)
        return time.perf_counter() - t0


_G = {}


def _init_worker(q, k, v):
    _G["qkv"] = (q, k, v)


def _oracle_unit_shared(args):
    q, k, v = _G["qkv"]
    return _oracle_unit((q, k, v) + tuple(args))


def _blas_name():
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                if i.get("user_api") == "blas"]
        return ", ".join(libs) or None
    except Exception:  # reporting only
        return None


def cpu_baseline(w, q64, k64, v64, budget_s=15.0):
    """Time the oracle on random 512-row blocks of random heads until about
    budget_s of wall time is used, over a process pool of one worker per core."""
    cores = len(os.sched_getaffinity(0))
    cores = max(1, min(cores, 16))
    rng = np.random.default_rng(12345)
    blk = 512
    n_blocks = (w.Nq + blk - 1) // blk
    off = w.N - w.Nq if w.causal else 0
    flops = 0.0
    done = 0
    t0 = time.perf_counter()
    ctx = __import__("multiprocessing").get_context("fork")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx, initializer=_init_worker,
                                initargs=(q64, k64, v64)) as ex:
        pending = set()
        submitted = 0

        def submit():
            nonlocal submitted
            b = int(rng.integers(w.B))
            h = int(rng.integers(w.H_q))
            r0 = int(rng.integers(n_blocks)) * blk
            rows = np.arange(r0, min(r0 + blk, w.Nq))
            f = ex.submit(_oracle_unit_shared, (b, h, rows, w.causal, w.sm_scale))
            vis = (rows + off + 1).sum() if w.causal else rows.size * w.N
            pending.add((f, 4.0 * w.D * float(vis)))
            submitted += 1

        for _ in range(2 * cores):
            submit()
        while pending:
            fs = {f for f, _ in pending}
            finished, _ = cf.wait(fs, return_when=cf.FIRST_COMPLETED)
            for item in list(pending):
                if item[0] in finished:
                    item[0].result()
                    flops += item[1]
                    done += 1
                    pending.discard(item)
                    if time.perf_counter() - t0 < budget_s:
                        submit()
    wall = time.perf_counter() - t0
    return {
        "value": round(flops / wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "numpy": np.__version__,
        "blas": _blas_name(),
        "kind": "oracle",
        "sample": (f"{done} blocks of {blk} query rows at random (b, h, row offset) of the "
                   f"{w.name} workload, float64 NumPy oracle, {cores} worker processes with "
                   f"one BLAS thread each, {wall:.1f} s wall; FLOPs counted as 4*D per visible "
                   f"(query, key) pair, the same convention as the GPU figure"),
    }


# ---------------------------------------------------------------- GPU timing
def make_step(ea, torch, w, qd, kd, vd, out, lse):
    """One call over the whole workload: attn_fwd for square workloads, else
    attn_fwd_splitkv with the library's split count and a preallocated workspace."""
    if w.N_q is None:
        return (lambda: ea.attn_fwd(qd, kd, vd, out, lse, is_causal=w.causal,
                                    sm_scale=w.sm_scale)), 1
    ns = ea.attn_splitkv_num_splits(w.B, w.H_q, w.H_kv, w.Nq, w.N, w.D, w.causal)
    nbytes = ea.attn_splitkv_workspace_size(w.B, w.H_q, w.Nq, w.D, ns)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=qd.device) if nbytes else None
    return (lambda: ea.attn_fwd_splitkv(qd, kd, vd, out, lse, is_causal=w.causal,
                                        sm_scale=w.sm_scale, n_splits=ns, workspace=ws)), ns


def auto_counts(torch, step, steps, warmup):
    """steps/warmup of None: enough launches for at least 100 ms of warm-up
    (the shader clock settles under load) and 200 ms of timed work, at least
    20 timed launches."""
    if steps is not None and warmup is not None:
        return steps, warmup
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    dt = max(time.perf_counter() - t0, 1e-6)
    return (steps if steps is not None else min(max(20, math.ceil(0.2 / dt)), 5000),
            warmup if warmup is not None else min(max(3, math.ceil(0.1 / dt)), 5000))


def time_workload(ea, torch, w, steps, warmup):
    dev = torch.device("cuda", 0)
    q, k, v = workloads.workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(w.q_shape(), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H_q, w.Nq), dtype=torch.float32, device=dev)
    step, n_splits = make_step(ea, torch, w, qd, kd, vd, out, lse)
    steps, warmup = auto_counts(torch, step, steps, warmup)
    for _ in range(warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    res = {"wall_ms_per_step": wall * 1e3 / steps, "event_ms": ev_ms, "n_splits": n_splits}
    return res, (q, k, v, out, lse)


def time_backward(ea, torch, w, steps, warmup):
    """attn_bwd over the whole workload: inputs Q, K, V, a seeded dO and this
    library's own forward output and LSE, all resident before timing."""
    dev = torch.device("cuda", 0)
    q, k, v = workloads.workload_inputs(w)
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 7919)
    dO = torch.randn(w.q_shape(), generator=g, dtype=torch.float32).to(torch.bfloat16)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), dO.to(dev)
    out, lse = ea.fwd_splitkv(qd, kd, vd, is_causal=w.causal, sm_scale=w.sm_scale, n_splits=1)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ns = max(ea.attn_bwd_num_splits(w.B, w.H_q, w.H_kv, w.Nq, w.N, w.D, w.causal), 1)
    ws = torch.empty((max(ea.attn_bwd_workspace_size(w.B, w.H_q, w.H_kv, w.Nq, w.N, w.D, w.causal, ns), 1),),
                     dtype=torch.uint8, device=dev)

    def step():
        ea.attn_bwd(qd, kd, vd, out, dod, lse, dq, dk, dv, is_causal=w.causal,
                    sm_scale=w.sm_scale, n_splits=ns, workspace=ws)
    steps, warmup = auto_counts(torch, step, steps, warmup)
    for _ in range(warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ({"wall_ms_per_step": wall * 1e3 / steps, "n_splits": ns,
             "event_ms": [s_.elapsed_time(e) for s_, e in zip(starts, ends)]},
            (q, k, v, dO, out.cpu(), dq.cpu(), dk.cpu(), dv.cpu()))


def _bwd_init(q64, k64, v64, d64, o64):
    _G["bwd"] = (q64, k64, v64, d64, o64)


def _bwd_task(args):
    from threadpoolctl import threadpool_limits
    import oracle
    kind, idx, sel, rows, causal, scale = args
    q64, k64, v64, d64, o64 = _G["bwd"]
    with threadpool_limits(1):
        if kind == "rows":
            return kind, idx, oracle.backward_rows(q64, k64, v64, d64, 0, idx, sel, is_causal=causal,
                                                   sm_scale=scale, out=o64)
        return kind, idx, oracle.backward_keys(q64, k64, v64, d64, 0, idx, sel, is_causal=causal,
                                               sm_scale=scale, out=o64, rows=rows)


def backward_parity(w, tensors):
    """Part of the CPU-baseline leg of --backward: dQ of sampled rows of every
    head of the first and last kv groups, and dK/dV of sampled keys of those
    groups summed over every query row, against the oracle's row and key
    entry points (key sums split over a process pool in 512-row blocks).
    Tolerance as the backward parity tests: |g - r| <= 2e-2 s + 2e-2 |r|, s the
    larger of the reference row's RMS, the sampled tensor's RMS and 1e-4."""
    q, k, v, dO, o, dq, dk, dv = tensors
    q64, k64, v64, d64, o64 = (workloads.to_float64(x) for x in (q, k, v, dO, o))
    N, G = w.N, w.H_q // w.H_kv
    rng = np.random.default_rng(w.seed + 1)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N // 2 - 1, N // 2, N - 129, N - 128,
                                      N - 65, N - 64, N - 2, N - 1], rng.choice(N, 6, replace=False)]))
    rows = rows[rows < w.Nq]
    keys = np.unique(np.concatenate([[0, 1, 127, 128, N // 2, N - 2, N - 1], rng.choice(N, 5, replace=False)]))
    groups = (0, w.H_kv - 1)
    tasks = [("rows", g * G + j, rows, None, w.causal, w.sm_scale) for g in groups for j in range(G)]
    tasks += [("keys", g, keys, np.arange(r0, min(r0 + 512, w.Nq)), w.causal, w.sm_scale)
              for g in groups for r0 in range(0, w.Nq, 512)]
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    t0 = time.perf_counter()
    ref_k = {g: np.zeros((keys.size, w.D)) for g in groups}
    ref_v = {g: np.zeros((keys.size, w.D)) for g in groups}
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    ok = True

    def check(name, got, ref):
        nonlocal ok
        g_ = got.double().numpy()
        rms = float(np.sqrt(np.mean(ref * ref)))
        sc = np.maximum(np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)), max(rms, 1e-4))
        err = np.abs(g_ - ref)
        ok = ok and bool(np.isfinite(g_).all()) and bool(np.all(err <= 2e-2 * sc + 2e-2 * np.abs(ref)))
        worst[name] = max(worst[name], float((err / (sc + np.abs(ref))).max()))

    ctx = __import__("multiprocessing").get_context("fork")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx, initializer=_bwd_init,
                                initargs=(q64, k64, v64, d64, o64)) as ex:
        for kind, idx, r in ex.map(_bwd_task, tasks):
            if kind == "rows":
                check("dQ", dq[0, idx, rows], r)
            else:
                ref_k[idx] += r[0]
                ref_v[idx] += r[1]
    for g in groups:
        check("dK", dk[0, g, keys], ref_k[g])
        check("dV", dv[0, g, keys], ref_v[g])
    return {"sampled_pass": ok, "dq_rows": int(rows.size) * len(groups) * G,
            "dkdv_keys": int(keys.size) * len(groups),
            "max_scaled_err": {k_: round(v_, 5) for k_, v_ in worst.items()},
            "wall_s": round(time.perf_counter() - t0, 1)}


def _parity_init(q, k, v, o, l):
    _G["parity"] = (q, k, v, o, l)


def _parity_head(args):
    from threadpoolctl import threadpool_limits
    import oracle
    b, h, causal, scale = args
    q, k, v, o, l = _G["parity"]
    with threadpool_limits(1):
        Or, Lr = oracle.attention_rows(q, k, v, b, h, np.arange(q.shape[2]), is_causal=causal,
                                       sm_scale=scale)
    og, lg = o[b, h].astype(np.float64), l[b, h].astype(np.float64)
    finite = bool(np.isfinite(og).all() and np.isfinite(lg).all())
    eo, el = np.abs(og - Or), np.abs(lg - Lr)
    ok = finite and bool(np.all(eo <= 2e-2 + 2e-2 * np.abs(Or))) and bool(np.all(el <= 1e-3))
    return ok, float(eo.max()), float(el.max())


def full_parity(w, q64, k64, v64, out, lse):
    """Part of the CPU-baseline leg: every row of the timed GPU output against
    the oracle on the same bf16 inputs, one (batch, head) per task over a
    process pool (one worker per core, at most 16)."""
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    t0 = time.perf_counter()
    ctx = __import__("multiprocessing").get_context("fork")
    tasks = [(b, h, w.causal, w.sm_scale) for b in range(w.B) for h in range(w.H_q)]
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx, initializer=_parity_init,
                                initargs=(q64, k64, v64, o, l)) as ex:
        res = list(ex.map(_parity_head, tasks))
    return {"all_rows_pass": all(r[0] for r in res), "rows": w.B * w.H_q * w.Nq,
            "max_abs_err_O": max(r[1] for r in res), "max_abs_err_LSE": max(r[2] for r in res),
            "wall_s": round(time.perf_counter() - t0, 1)}


def time_mla(ea, torch, name, mw, steps, warmup):
    """MLA decode (absorbed): the three steps timed together, plus the latent
    core alone; core FLOPs 2*(2*512+64) per visible (token, head, key).
    steps/warmup None: time-based counts (auto_counts)."""
    dev = torch.device("cuda", 0)
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(mw.B, mw.H, mw.S, mw.T, mw.seed)
    kv = torch.cat([c_kv, k_pe], -1).contiguous().to(dev)
    qn, qp, wk, wv = q_nope.to(dev), q_pe.to(dev), W_uk.to(dev), W_uv.to(dev)
    q_lat = torch.empty((mw.B, mw.H, mw.S, 576), dtype=torch.bfloat16, device=dev)
    out_lat = torch.empty((mw.B, mw.H, mw.S, 512), dtype=torch.bfloat16, device=dev)
    lse_m = torch.empty((mw.B, mw.H, mw.S), dtype=torch.float32, device=dev)
    out_m = torch.empty((mw.B, mw.H, mw.S, mw.d_v), dtype=torch.bfloat16, device=dev)
    ns = ea.attn_mla_num_splits(mw.B, mw.H, mw.S, mw.T, mw.causal)
    nb = ea.attn_mla_workspace_size(mw.B, mw.H, mw.S, ns)
    ws_m = torch.empty((max(nb, 1),), dtype=torch.uint8, device=dev)

    def core():
        ea.attn_mla_decode(q_lat, kv, out_lat, lse_m, mw.sm_scale, is_causal=mw.causal,
                           n_splits=ns, workspace=ws_m)

    def full():
        ea.mla_absorb_q(qn, qp, wk, q_lat)
        core()
        ea.mla_up_project(out_lat, wv, out_m)
    res_t = {}
    for label, fn in (("core", core), ("full", full)):
        n_steps, n_warm = auto_counts(torch, fn, steps, warmup)
        for _ in range(n_warm):
            fn()
        ev = []
        for _ in range(n_steps):
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            fn()
            e_.record()
            ev.append((s_, e_))
        torch.cuda.synchronize()
        res_t[label] = float(np.median([a.elapsed_time(b_) for a, b_ in ev]))
    t = res_t["core"]
    log(f"[mla] {name:22s} splits {ns:3d}  core {t * 1e3:8.1f} us  "
        f"{mw.core_bytes() / t / 1e6:7.0f} GB/s  {mw.core_flops() / t / 1e9:7.1f} TFLOP/s   "
        f"absorb+core+up {res_t['full'] * 1e3:8.1f} us")
    if steps is None:
        return None
    return {"core_ms": t, "step_ms": res_t["full"], "n_splits": ns,
            "tensors": (q_lat, kv, out_lat, lse_m)}


def mla_parity(mw, tensors):
    """Part of the CPU-baseline leg of --mla: the latent core's output and LSE
    against the oracle on the core's own inputs (the absorbed queries this run produced, the latent cache), for
    every head of the first and the last batch element; tolerance as the MLA
    GPU tests (2e-2 absolute plus 2e-2 relative on O, 1e-3 on the LSE)."""
    import oracle
    q_lat, kv, out_lat, lse_m = tensors
    t0 = time.perf_counter()
    worst_o = worst_l = 0.0
    ok = True
    for b in sorted({0, mw.B - 1}):
        q64 = q_lat[b:b + 1].float().cpu().numpy().astype(np.float64)
        kv64 = kv[b:b + 1].float().cpu().numpy().astype(np.float64)
        O, L = oracle.mla_latent_attention(q64, kv64, mw.d_c, is_causal=mw.causal, sm_scale=mw.sm_scale)
        o = out_lat[b:b + 1].float().cpu().numpy().astype(np.float64)
        l = lse_m[b:b + 1].cpu().numpy().astype(np.float64)
        err_o, err_l = np.abs(o - O), np.abs(l - L)
        ok &= bool(np.isfinite(o).all() and np.isfinite(l).all())
        ok &= bool((err_o <= 2e-2 + 2e-2 * np.abs(O)).all()) and bool(err_l.max() <= 1e-3)
        worst_o, worst_l = max(worst_o, float(err_o.max())), max(worst_l, float(err_l.max()))
    return {"sampled_pass": ok, "batch_elements": sorted({0, mw.B - 1}), "heads": mw.H,
            "max_abs_err_O": worst_o, "max_abs_err_LSE": worst_l,
            "wall_s": round(time.perf_counter() - t0, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--sweep", action="store_true",
                    help="also time every workload and print a table to stderr")
    ap.add_argument("--mla-sweep", action="store_true",
                    help="time the MLA decode workloads and print a table to stderr, then exit")
    ap.add_argument("--backward-sweep", action="store_true",
                    help="time attn_bwd on the square workloads and print a table to stderr, then exit")
    ap.add_argument("--backward", action="store_true",
                    help="time attn_bwd on --workload only (--steps, --warmup), print one line to stderr, exit")
    ap.add_argument("--mla", default=None, choices=sorted(workloads.MLA_WORKLOADS),
                    help="time one MLA decode workload (--steps, --warmup), print one line to stderr, exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 512 MiB three times "
                         "(reference for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this attention forward has no multi-GPU path "
              "(sharding by batch or kv-head group needs no communication and is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_02_amd as ea
    ea.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    if args.mla_sweep:
        for name, mw in workloads.MLA_WORKLOADS.items():
            time_mla(ea, torch, name, mw, None, None)
        return
    if args.mla:
        # one MLA workload: the latent core (split pass + merge) against the
        # roofline that binds it, one JSON line
        mw = workloads.MLA_WORKLOADS[args.mla]
        r = time_mla(ea, torch, args.mla, mw, args.steps, args.warmup)
        t_s = r["core_ms"] * 1e-3
        gbs, tfs = mw.core_bytes() / t_s / 1e9, mw.core_flops() / t_s / 1e12
        hbm_frac, mfma_frac = gbs / PEAK_HBM_GBS, tfs / PEAK_BF16_TFLOPS
        traffic = read_profile(f"attn_{args.mla}_hbm_traffic.md", "core_hbm_bytes_per_launch", MLA_SOURCES)
        if hbm_frac >= mfma_frac:
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(hbm_frac, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tfs, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(mfma_frac, 4)}
        roof.update({"traffic": traffic, "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
                     "kernel": "attn_mla_decode (latent-core split pass + merge)",
                     "median_launch_ms": round(r["core_ms"], 5), "n_splits": r["n_splits"],
                     "algorithmic_bytes_per_launch": mw.core_bytes(),
                     "algorithmic_flops_per_launch": mw.core_flops()})
        parity = None if args.no_cpu_baseline else mla_parity(mw, r["tensors"])
        print(json.dumps({
            "metric": "MLA absorbed decode: latent core time against its binding roofline",
            "value": round(r["core_ms"] * 1e3, 2), "unit": "us", "higher_is_better": False,
            "step_us": round(r["step_ms"] * 1e3, 2), "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": mw.name, "B": mw.B, "H": mw.H, "S": mw.S, "T": mw.T, "d_c": mw.d_c,
                       "d_r": mw.d_r, "causal": mw.causal, "seed": mw.seed},
            "roofline": roof, "parity": parity}), flush=True)
        return

    if args.backward:
        # one workload's attn_bwd alone, one JSON line (counter runs: --steps 2
        # --warmup 1 --no-cpu-baseline)
        w = workloads.WORKLOADS[args.workload]
        r, tensors = time_backward(ea, torch, w, args.steps, args.warmup)
        ev = r["event_ms"]
        avg = float(np.mean(ev))
        flops = 2.5 * w.flops()   # five products of 2*D per visible (query, key) pair
        nbytes = w.bwd_algorithmic_bytes()
        log(f"[bwd] {w.name:24s} median {float(np.median(ev)):9.4f} ms  min {min(ev):9.4f} ms  "
            f"{flops / (avg * 1e-3) / 1e12:8.1f} TFLOP/s  splits {r['n_splits']}  ({len(ev)} launches)")
        parity = None
        if not args.no_cpu_baseline:
            log("[bwd] oracle: sampled dQ rows and dK/dV keys")
            parity = backward_parity(w, tensors)
            log(f"[bwd] parity {parity}")
        achieved = flops / (avg * 1e-3) / 1e12
        traffic = read_profile(f"attn_bwd_{w.name}_hbm_traffic.md", "hbm_bytes_per_launch", BWD_SOURCES)
        busy = read_profile(f"attn_bwd_{w.name}_hbm_traffic.md", "mfma_busy_frac", BWD_SOURCES)
        print(json.dumps({
            "metric": "attention bwd TFLOPS (dQ, dK, dV; 2.5x the forward FLOPs) and % of MI355X bf16 MFMA peak",
            "value": round(flops / (r["wall_ms_per_step"] * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": len(ev), "ms_per_step": round(r["wall_ms_per_step"], 4),
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N": w.N,
                       "N_q": w.Nq, "D": w.D, "causal": w.causal, "seed": w.seed},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic, "mfma_busy": busy,
                         "kernel": "attn_bwd (prep, dK/dV and dQ kernels)",
                         "avg_launch_ms": round(avg, 4), "median_launch_ms": round(float(np.median(ev)), 4),
                         "n_splits": r["n_splits"], "algorithmic_flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": nbytes},
            "parity": parity}), flush=True)
        return

    if args.backward_sweep:
        # backward FLOPs: the five products of 2*D per visible (query, key) pair
        # (S recomputed, dP, dV, dK, dQ), i.e. 2.5x the forward's count
        for name, ww in workloads.WORKLOADS.items():
            if ww.N_q is not None and name != "chunk_gqa4_q512_n8192":
                continue
            r, _ = time_backward(ea, torch, ww, None, None)
            e = float(np.median(r["event_ms"]))
            tf = 2.5 * ww.flops() / (e * 1e-3) / 1e12
            log(f"[bwd] {name:24s} median {e:9.4f} ms  min {min(r['event_ms']):9.4f} ms  "
                f"{tf:8.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:5.1f}%)  splits {r['n_splits']}  "
                f"({len(r['event_ms'])} launches)")
        return

    w = workloads.WORKLOADS[args.workload]
    log(f"[bench] timing {w.name}: steps={args.steps} warmup={args.warmup}")
    res, (q, k, v, out, lse) = time_workload(ea, torch, w, args.steps, args.warmup)
    ev = res["event_ms"]
    avg_ms = float(np.mean(ev))
    flops = w.flops()
    value = flops / (res["wall_ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    log(f"[bench] wall {res['wall_ms_per_step']:.3f} ms/step, event avg {avg_ms:.3f} ms "
        f"(min {min(ev):.3f}, median {float(np.median(ev)):.3f}), {achieved:.1f} TFLOP/s")

    if args.sweep:
        for name, ww in workloads.WORKLOADS.items():
            r, _ = time_workload(ea, torch, ww, None, None)
            e = r["event_ms"]
            tf = ww.flops() / (float(np.median(e)) * 1e-3) / 1e12
            gbs = ww.algorithmic_bytes() / (float(np.median(e)) * 1e-3) / 1e9
            log(f"[sweep] {name:24s} median {float(np.median(e)):9.4f} ms  min {min(e):9.4f} ms  "
                f"{tf:8.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:5.1f}%)  {gbs:7.0f} GB/s "
                f"({100 * gbs / PEAK_HBM_GBS:5.1f}%)  splits {r['n_splits']}  ({len(e)} launches)")

    cpu = parity = None
    if not args.no_cpu_baseline:
        # the only part of the benchmark that runs the oracle
        log("[bench] oracle: every row of the output (parity), then a bounded sample (cpu_baseline)")
        q64, k64, v64 = (workloads.to_float64(t) for t in (q, k, v))
        parity = full_parity(w, q64, k64, v64, out, lse)
        log(f"[bench] parity {parity}")
        cpu = cpu_baseline(w, q64, k64, v64, budget_s=args.cpu_budget)
        log(f"[bench] cpu_baseline {cpu}")

    traffic = read_traffic(w.name)
    nbytes = w.algorithmic_bytes()
    if flops / nbytes >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        clock = read_clock(w.name)
        if clock is not None:
            # the same dense bf16 MFMA rate (4096 flop per clock per CU, 256
            # CUs) at the clock the chip held during this kernel
            peak_clk = MFMA_FLOP_PER_CLK * clock * 1e9 / 1e12
            roofline.update({"clock_ghz": clock, "peak_at_clock": round(peak_clk, 1),
                             "frac_at_clock": round(achieved / peak_clk, 4)})
        busy = read_mfma_busy(w.name)
        if busy is not None:
            roofline["mfma_busy"] = busy
    else:
        # below the ridge (decode): bytes moved, not FLOPs, bound the kernel
        gbs = nbytes / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    kernel = "attn_fwd_kernel" if res["n_splits"] == 1 else "attn_fwd_kernel split pass + attn_merge_kernel"
    roofline.update({"traffic": traffic, "kernel": kernel, "avg_launch_ms": round(avg_ms, 4),
                     "median_launch_ms": round(float(np.median(ev)), 4), "min_launch_ms": round(min(ev), 4),
                     "n_splits": res["n_splits"],
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes})
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N": w.N,
                   "N_q": w.Nq, "D": w.D, "causal": w.causal, "seed": w.seed},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
