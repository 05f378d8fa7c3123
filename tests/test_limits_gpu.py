"""GPU parity at the largest key count the ABI admits.

One kv head of N_kv = 2^23 keys at D = 128 is exactly 2^31 bytes, the limit of
the 32-bit byte offsets the kernels use within a head (SIZE_OVERFLOW above
it).  The decode shapes run here touch every key of that head: N_q = 1
(one pass, n_splits = 1, and the library's split count) and N_q = 4 with the
bottom-right causal mask.  H_q = 4 query heads share the one kv head.

Inputs are drawn on the device from a seeded generator (2 GiB each for K and
V) and copied to the host for the reference.  The float64 oracle cannot hold
the head at once, so the reference takes it in chunks of 2^18 keys: the
oracle's attention over each chunk, combined with the oracle's split-T merge
(merge_partials, pinned against the unsplit oracle).  This is the same
definition, evaluated piecewise; each chunk is converted once and serves every
head and row.  Tolerances are the forward's: O within 2e-2 + 2e-2 |ref|, LSE
within 1e-3.

The last test forces a 33-way key split over 17 x 131072 = 2228224 output
rows: more than 2^21 rows, so the merge (1024-thread blocks at that split
count) runs as two launches of at most 2^31 work-items.  Sampled rows on both
sides of the launch boundary go to the oracle; every row must also agree with
the unsplit pass of the library within the same tolerance.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

N_KV = 1 << 23
D = 128
H_Q = 4
CHUNK = 1 << 18
SEED = 14000


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_02_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def kv():
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(SEED)
    k = torch.randn((1, 1, N_KV, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((1, 1, N_KV, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    return k, v, k.cpu(), v.cpu()


def _queries(N_q, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn((1, H_Q, N_q, D), generator=g, dtype=torch.float32).to(torch.bfloat16)


def _reference(q, k_cpu, v_cpu, causal, scale):
    """(O [H_Q, N_q, D], LSE [H_Q, N_q]) by chunks of keys and the oracle merge."""
    N_q = q.shape[2]
    q64 = workloads.to_float64(q)
    o_parts = {(h, i): [] for h in range(H_Q) for i in range(N_q)}
    l_parts = {(h, i): [] for h in range(H_Q) for i in range(N_q)}
    for c0 in range(0, N_KV, CHUNK):
        c1 = min(c0 + CHUNK, N_KV)
        k64 = workloads.to_float64(k_cpu[:, :, c0:c1])
        v64 = workloads.to_float64(v_cpu[:, :, c0:c1])
        # rows that see the whole chunk: one oracle call for all of them
        full = [i for i in range(N_q) if not causal or i + N_KV - N_q >= c1 - 1]
        if full:
            O, L = oracle.attention_forward(q64[:, :, full], k64, v64, is_causal=False, sm_scale=scale)
            for j, i in enumerate(full):
                for h in range(H_Q):
                    o_parts[(h, i)].append(O[0, h, j])
                    l_parts[(h, i)].append(L[0, h, j])
        for i in range(N_q):
            if i in full:
                continue
            n = i + N_KV - N_q + 1 - c0  # keys of this chunk the row sees
            if n <= 0:
                continue
            O, L = oracle.attention_forward(q64[:, :, i:i + 1], k64[:, :, :n], v64[:, :, :n],
                                            is_causal=False, sm_scale=scale)
            for h in range(H_Q):
                o_parts[(h, i)].append(O[0, h, 0])
                l_parts[(h, i)].append(L[0, h, 0])
    O = np.empty((H_Q, N_q, D))
    L = np.empty((H_Q, N_q))
    for (h, i), parts in o_parts.items():
        O[h, i], L[h, i] = oracle.merge_partials(np.stack(parts), np.array(l_parts[(h, i)]))
    return O, L


def _check(out, lse, O, L, what):
    o = out.cpu().to(torch.float64).numpy()[0]
    l = lse.cpu().to(torch.float64).numpy()[0]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite"
    err = np.abs(o - O)
    bad = err > 2e-2 + 2e-2 * np.abs(O)
    assert not bad.any(), f"{what}: {int(bad.sum())} O elements out of tolerance, max {err.max():.3e}"
    assert np.abs(l - L).max() <= 1e-3, f"{what}: LSE error {np.abs(l - L).max():.3e}"


def test_decode_at_max_keys(ea, kv):
    """N_q = 1, non-causal: the single pass walks all 2^23 keys in one
    workgroup; the split pass divides them by the library's choice."""
    k, v, k_cpu, v_cpu = kv
    dev = k.device
    scale = 1.0 / math.sqrt(D)
    q = _queries(1, SEED + 1)
    O, L = _reference(q, k_cpu, v_cpu, False, scale)
    print("[limits] decode N_kv=2^23: reference done", flush=True)
    for ns in (1, 0):
        out, lse = ea.fwd_splitkv(q.to(dev), k, v, is_causal=False, sm_scale=scale, n_splits=ns)
        torch.cuda.synchronize()
        _check(out, lse, O, L, f"attn_fwd_splitkv n_splits={ns}")


def test_causal_suffix_at_max_keys(ea, kv):
    """N_q = 4 bottom-right causal: row i sees keys 0 .. 2^23 - 4 + i."""
    k, v, k_cpu, v_cpu = kv
    dev = k.device
    scale = 1.0 / math.sqrt(D)
    q = _queries(4, SEED + 2)
    O, L = _reference(q, k_cpu, v_cpu, True, scale)
    print("[limits] causal N_q=4 N_kv=2^23: reference done", flush=True)
    for ns in (0, 1):
        out, lse = ea.fwd_splitkv(q.to(dev), k, v, is_causal=True, sm_scale=scale, n_splits=ns)
        torch.cuda.synchronize()
        _check(out, lse, O, L, f"attn_fwd_splitkv n_splits={ns}")


def test_split_merge_over_many_rows(ea):
    """2228224 rows, 33 forced key splits: the merge's second launch (rows
    from 2^21 on) must cover its rows exactly like the first."""
    B, H, N_q, N_kv = 1, 17, 131072, 33 * 64
    dev = torch.device("cuda", 0)
    scale = 1.0 / math.sqrt(D)
    g = torch.Generator(device=dev)
    g.manual_seed(SEED + 3)
    q = torch.randn((B, H, N_q, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, H, N_kv, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, H, N_kv, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    print(f"[limits] split merge rows={B * H * N_q} n_splits=33", flush=True)
    out, lse = ea.fwd_splitkv(q, k, v, is_causal=False, sm_scale=scale, n_splits=33)
    torch.cuda.synchronize()
    out1, lse1 = ea.fwd_splitkv(q, k, v, is_causal=False, sm_scale=scale, n_splits=1)
    torch.cuda.synchronize()
    # flattened row r = h * N_q + i; the second merge launch starts at r = 2^21
    boundary = 1 << 21
    rows = sorted({0, boundary - 1, boundary, boundary + 1, B * H * N_q - 1,
                   *range(boundary - 64, boundary + 64, 5),
                   *np.random.default_rng(SEED + 4).integers(0, B * H * N_q, 48).tolist()})
    k_cpu, v_cpu, q_cpu = k.cpu(), v.cpu(), q.cpu()
    o_g = out.cpu().to(torch.float64).numpy()[0]
    l_g = lse.cpu().to(torch.float64).numpy()[0]
    for h in sorted({r // N_q for r in rows}):
        idx = [r % N_q for r in rows if r // N_q == h]
        O, L = oracle.attention_forward(workloads.to_float64(q_cpu[:, h:h + 1, idx]),
                                        workloads.to_float64(k_cpu[:, h:h + 1]),
                                        workloads.to_float64(v_cpu[:, h:h + 1]),
                                        is_causal=False, sm_scale=scale)
        _check(torch.from_numpy(o_g[h:h + 1, idx])[None], torch.from_numpy(l_g[h:h + 1, idx])[None],
               O[0], L[0], f"n_splits=33 head {h} rows {idx[:3]}...")
    # every row against the unsplit pass
    err = (out.float() - out1.float()).abs()
    bad = err > 2e-2 + 2e-2 * out1.float().abs()
    assert not bool(bad.any()), f"{int(bad.sum())} elements differ from the unsplit pass"
    assert float((lse - lse1).abs().max()) <= 1e-3
