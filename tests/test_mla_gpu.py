"""GPU parity of the MLA decode path (absorbed form) against the float64 CPU
oracle.

Inputs are the seeded recipe of workloads.make_mla_inputs (DeepSeek-V3 shapes
of page "Attention Kernel 实现与正确性验证", section 2.3, or smaller).  Each
step is checked against the oracle on the same bf16 operands, and the whole
pipeline against the oracle's naive form (keys and values reconstructed per
head, the definition):
  * latent core: out_lat within 2e-2 + 2e-2 |ref|, LSE within 1e-3;
  * projections and the pipeline: the forward's allclose made scale-free,
    |y - ref| <= 2e-2 rms(ref) + 2e-2 |ref|, because the absorbed query and
    the latent output are rounded to bf16 between the steps.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_02_amd as m
    m.load_library()
    return m


def _dev():
    return torch.device("cuda", 0)


def _f64(t):
    return workloads.to_float64(t)


def _check_attn(o, l, O_ref, L_ref, what):
    o = o.to(torch.float64).numpy()
    l = l.to(torch.float64).numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite"
    err = np.abs(o - O_ref)
    bad = err > 2e-2 + 2e-2 * np.abs(O_ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} out of tolerance, max {err.max():.3e}"
    assert np.abs(l - L_ref).max() <= 1e-3, f"{what}: lse err {np.abs(l - L_ref).max():.3e}"


def _check_scaled(y, ref, what):
    y = y.to(torch.float64).numpy()
    assert np.all(np.isfinite(y)), f"{what}: non-finite"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(y - ref)
    bad = err > 2e-2 * rms + 2e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} out of tolerance, max {err.max():.3e} rms {rms:.3e}"


def _latent_inputs(B, H, S, T, seed):
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(B, H, S, T, seed)
    kv = torch.cat([c_kv, k_pe], dim=-1).contiguous()
    q_lat = torch.from_numpy(oracle.mla_absorb_q(_f64(q_nope), _f64(q_pe), _f64(W_uk))).to(torch.bfloat16)
    return q_lat, kv


def _run_core(ea, q_lat, kv, scale, causal, n_splits):
    dev = _dev()
    B, H, S, _ = q_lat.shape
    T = kv.shape[1]
    out = torch.full((B, H, S, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=dev)
    ns = n_splits if n_splits > 0 else ea.attn_mla_num_splits(B, H, S, T, causal)
    nbytes = ea.attn_mla_workspace_size(B, H, S, ns)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev) if nbytes else None
    ea.attn_mla_decode(q_lat.to(dev), kv.to(dev), out, lse, scale, is_causal=causal,
                       n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_splits", [1, 3, 0])
def test_latent_core(ea, T, causal, n_splits):
    B, H, S = 2, 16, 1
    q_lat, kv = _latent_inputs(B, H, S, T, seed=13000 + T)
    sc = 1 / math.sqrt(192)
    o, l = _run_core(ea, q_lat, kv, sc, causal, n_splits)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=causal, sm_scale=sc)
    _check_attn(o, l, O, L, f"T{T} c{int(causal)} s{n_splits}")


@pytest.mark.parametrize("n_splits", [7, 24, 100, 256])
def test_latent_core_merge_shapes(ea, n_splits):
    """Split counts that take each merge launch shape at D = 512: 256-thread
    blocks (up to 8 splits), 1024 with 4 splits per thread (up to 32), 1024
    with 16 (up to 128), and the two-pass merge beyond."""
    B, H, S, T = 2, 16, 1, 5000
    q_lat, kv = _latent_inputs(B, H, S, T, seed=13050 + n_splits)
    sc = 1 / math.sqrt(192)
    o, l = _run_core(ea, q_lat, kv, sc, True, n_splits)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=True, sm_scale=sc)
    _check_attn(o, l, O, L, f"T{T} s{n_splits}")


@pytest.mark.parametrize("H,S,T", [(128, 1, 300), (128, 2, 129), (7, 5, 70), (3, 4, 4), (40, 3, 65)])
@pytest.mark.parametrize("n_splits", [1, 4])
def test_latent_core_heads_and_tokens(ea, H, S, T, n_splits):
    """Pair blocks that mix query tokens, head counts that do not divide 32,
    several causal query tokens (bottom-right)."""
    q_lat, kv = _latent_inputs(1, H, S, T, seed=13100 + H + S)
    sc = 1 / math.sqrt(192)
    for causal in (False, True):
        o, l = _run_core(ea, q_lat, kv, sc, causal, n_splits)
        O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=causal, sm_scale=sc)
        _check_attn(o, l, O, L, f"H{H} S{S} T{T} c{int(causal)}")


# Shapes whose workgroups before any split (B times ceil(S H / 128)) number at
# least an eighth of the CUs: on a 256-CU MI355X the latent core runs them
# with its sixteen-pair kernel (128 pairs per workgroup), the others with the
# four-wave kernel (64 pairs).
@pytest.mark.parametrize("B,H,S,T,causal,n_splits,scale", [
    (32, 16, 3, 65, True, 1, 0.07), (32, 16, 3, 65, False, 3, 0.07), (32, 128, 1, 31, True, 0, 0.07),
    (40, 128, 2, 129, True, 0, 0.07), (33, 7, 5, 1000, True, 7, 0.07), (33, 7, 5, 1000, False, 0, -0.05),
    (32, 40, 3, 300, True, 2, 0.3)])
def test_latent_core_sixteen_pair_shapes(ea, B, H, S, T, causal, n_splits, scale):
    """Ragged cache ends, several pair blocks per batch element, bottom-right
    causal query tokens, forced and library split counts, grids that are and
    are not a multiple of the 8 XCDs, a negative scale."""
    q_lat, kv = _latent_inputs(B, H, S, T, seed=13700 + B + H + S + T)
    o, l = _run_core(ea, q_lat, kv, scale, causal, n_splits)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=causal, sm_scale=scale)
    _check_attn(o, l, O, L, f"B{B} H{H} S{S} T{T} c{int(causal)} s{n_splits}")


@pytest.mark.parametrize("B", [1, 32])
@pytest.mark.parametrize("n_splits", [1, 2])
def test_latent_core_growing_scores(ea, n_splits, B):
    """Cache rows whose norm grows along T: the running max of a row rises
    by more than the lazy-rescale slack (8 in log2 units) on many tiles, so
    the accumulators are rescaled again and again.  The inputs are checked
    on the CPU to force at least 4 such rises for every row (the max over a
    32-key tile against the largest max so far plus 8, in fp64)."""
    H, S, T = 64, 1, 1024
    q_lat, kv = _latent_inputs(B, H, S, T, seed=13300)
    # the steeper ramp at B = 32 gives every one of its rows the 4 rises too
    ramp = torch.linspace(0.1, 6.0 if B == 1 else 8.0, T).view(1, T, 1)
    kv = (kv.float() * ramp).to(torch.bfloat16)
    sc = 0.3
    s2 = np.einsum("bhsd,btd->bhst", _f64(q_lat), _f64(kv)) * sc / math.log(2)
    tile_max = s2.reshape(B, H, S, T // 32, 32).max(-1)
    rises = np.zeros((B, H, S), dtype=np.int64)
    m_used = tile_max[..., 0]
    for t in range(1, T // 32):
        up = tile_max[..., t] > m_used + 8
        rises += up
        m_used = np.where(up, tile_max[..., t], m_used)
    assert rises.min() >= 4, f"inputs force too few rescales: min {rises.min()}"
    o, l = _run_core(ea, q_lat, kv, sc, False, n_splits)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=False, sm_scale=sc)
    _check_attn(o, l, O, L, f"growing scores s{n_splits}")


@pytest.mark.parametrize("scale", [0.0, -0.05, 0.3])
def test_latent_core_scales(ea, scale):
    q_lat, kv = _latent_inputs(1, 32, 1, 500, seed=13200)
    o, l = _run_core(ea, q_lat, kv, scale, True, 3)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=True, sm_scale=scale)
    _check_attn(o, l, O, L, f"scale {scale}")


def test_projections(ea):
    dev = _dev()
    B, H, S = 3, 8, 2
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(B, H, S, 10, 13300)
    q_lat = torch.empty((B, H, S, 576), dtype=torch.bfloat16, device=dev)
    ea.mla_absorb_q(q_nope.to(dev), q_pe.to(dev), W_uk.to(dev), q_lat)
    ref = oracle.mla_absorb_q(_f64(q_nope), _f64(q_pe), _f64(W_uk))
    _check_scaled(q_lat.cpu()[..., :512], ref[..., :512], "absorb")
    assert torch.equal(q_lat.cpu()[..., 512:].view(torch.int16), q_pe.view(torch.int16)), "q_pe copy"
    g = torch.Generator(device="cpu")
    g.manual_seed(13301)
    x = torch.randn((B, H, S, 512), generator=g).to(torch.bfloat16)
    y = torch.empty((B, H, S, 128), dtype=torch.bfloat16, device=dev)
    ea.mla_up_project(x.to(dev), W_uv.to(dev), y)
    _check_scaled(y.cpu(), oracle.mla_up_project(_f64(x), _f64(W_uv)), "up")


@pytest.mark.parametrize("offset", [1, 0])
@pytest.mark.parametrize("d_nope,B,H,S", [(128, 1, 128, 1), (128, 32, 128, 1), (1, 2, 3, 1), (17, 5, 4, 7),
                                           (64, 3, 8, 12), (100, 1, 6, 70), (192, 2, 4, 33),
                                           (256, 4, 5, 9), (8, 3, 2, 40), (24, 2, 3, 5)])
def test_absorb_shapes(ea, d_nope, B, H, S, offset):
    """mla_absorb_q over d_nope 1..256 (zero-padded to whole k-steps inside),
    row counts spanning several 32-row blocks with a ragged last one, and a
    q_nope that starts 2 bytes past a 16-byte boundary (offset 1: the
    value-by-value query loads) or on one (offset 0: 16-byte query loads
    where d_nope is a multiple of 8)."""
    dev = _dev()
    g = torch.Generator(device="cpu")
    g.manual_seed(13400 + d_nope + B * H * S)
    q_nope = torch.randn((B, H, S, d_nope), generator=g).to(torch.bfloat16)
    q_pe = torch.randn((B, H, S, 64), generator=g).to(torch.bfloat16)
    W_uk = (torch.randn((H, d_nope, 512), generator=g) / math.sqrt(d_nope)).to(torch.bfloat16)
    buf = torch.empty(q_nope.numel() + 8, dtype=torch.bfloat16, device=dev)
    assert buf.data_ptr() % 16 == 0
    qn = buf[offset:offset + q_nope.numel()].view(q_nope.shape)
    qn.copy_(q_nope.to(dev))
    q_lat = torch.full((B, H, S, 576), float("nan"), dtype=torch.bfloat16, device=dev)
    ea.mla_absorb_q(qn, q_pe.to(dev), W_uk.to(dev), q_lat)
    torch.cuda.synchronize()
    ref = oracle.mla_absorb_q(_f64(q_nope), _f64(q_pe), _f64(W_uk))
    _check_scaled(q_lat.cpu()[..., :512], ref[..., :512], f"absorb d{d_nope}")
    assert torch.equal(q_lat.cpu()[..., 512:].view(torch.int16), q_pe.view(torch.int16)), "q_pe copy"


@pytest.mark.parametrize("B,H,S,T,causal", [(2, 16, 1, 200, True), (1, 128, 1, 300, True),
                                            (1, 8, 3, 50, True), (33, 4, 1, 40, False)])
def test_pipeline_against_naive(ea, B, H, S, T, causal):
    """absorb -> latent core -> up-projection against the naive definition."""
    dev = _dev()
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(B, H, S, T, 13400 + B + H)
    kv = torch.cat([c_kv, k_pe], dim=-1).contiguous()
    out, lse = ea.mla_decode(q_nope.to(dev), q_pe.to(dev), kv.to(dev), W_uk.to(dev), W_uv.to(dev),
                             is_causal=causal)
    torch.cuda.synchronize()
    ref = oracle.mla_naive(_f64(c_kv), _f64(k_pe), _f64(q_nope), _f64(q_pe), _f64(W_uk), _f64(W_uv),
                           is_causal=causal, sm_scale=1 / math.sqrt(192))
    _check_scaled(out.cpu(), ref, f"pipeline B{B} H{H} S{S} T{T}")


@pytest.mark.parametrize("name", sorted(workloads.MLA_WORKLOADS))
def test_mla_workloads(ea, name):
    """The decode workloads at full size: every head of the first and last
    batch element, pipeline against the oracle's absorbed form (pinned equal to
    the naive form)."""
    w = workloads.MLA_WORKLOADS[name]
    dev = _dev()
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(w.B, w.H, w.S, w.T, w.seed)
    kv = torch.cat([c_kv, k_pe], dim=-1).contiguous()
    out, _ = ea.mla_decode(q_nope.to(dev), q_pe.to(dev), kv.to(dev), W_uk.to(dev), W_uv.to(dev),
                           is_causal=w.causal)
    torch.cuda.synchronize()
    for b in sorted({0, w.B - 1}):
        sl = slice(b, b + 1)
        ref = oracle.mla_absorbed(_f64(c_kv[sl]), _f64(k_pe[sl]), _f64(q_nope[sl]), _f64(q_pe[sl]),
                                  _f64(W_uk), _f64(W_uv), is_causal=w.causal, sm_scale=w.sm_scale)
        _check_scaled(out.cpu()[sl], ref, f"{name} b{b}")


def test_mla_deterministic(ea):
    q_lat, kv = _latent_inputs(1, 128, 1, 3000, seed=13500)
    a = _run_core(ea, q_lat, kv, 0.07, True, 0)
    b = _run_core(ea, q_lat, kv, 0.07, True, 0)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def _draw_mla_cases(seed: int = 20261203, n: int = 10):
    """Seeded random MLA problems: batch, head count (not only multiples of
    32), query tokens per step (bottom-right causal when S > 1), cache length
    and split count (the library's or a forced one)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.choice([1, 5, 16, 40, 128]))
        S = int(rng.integers(1, 5))
        T = int(rng.integers(S, 2000))
        causal = bool(rng.random() < 0.6)
        n_splits = int(rng.choice([0, 1, 2, 5, 17]))
        cases.append((B, H, S, T, causal, n_splits, 13600 + i))
    return cases


@pytest.mark.parametrize("B,H,S,T,causal,n_splits,seed", _draw_mla_cases())
def test_mla_random_shapes(ea, B, H, S, T, causal, n_splits, seed):
    """The latent core against the oracle on a seeded random shape, then the
    whole pipeline (absorb, core with the library's splits, up-projection)
    against the naive definition on the same draw."""
    sc = 1 / math.sqrt(192)
    q_lat, kv = _latent_inputs(B, H, S, T, seed)
    o, l = _run_core(ea, q_lat, kv, sc, causal, n_splits)
    O, L = oracle.mla_latent_attention(_f64(q_lat), _f64(kv), 512, is_causal=causal, sm_scale=sc)
    _check_attn(o, l, O, L, f"core B{B} H{H} S{S} T{T} c{int(causal)} s{n_splits}")
    dev = _dev()
    c_kv, k_pe, q_nope, q_pe, W_uk, W_uv = workloads.make_mla_inputs(B, H, S, T, seed)
    kvd = torch.cat([c_kv, k_pe], dim=-1).contiguous()
    out, _ = ea.mla_decode(q_nope.to(dev), q_pe.to(dev), kvd.to(dev), W_uk.to(dev), W_uv.to(dev),
                           is_causal=causal)
    torch.cuda.synchronize()
    ref = oracle.mla_naive(_f64(c_kv), _f64(k_pe), _f64(q_nope), _f64(q_pe), _f64(W_uk), _f64(W_uv),
                           is_causal=causal, sm_scale=sc)
    _check_scaled(out.cpu(), ref, f"pipeline B{B} H{H} S{S} T{T} c{int(causal)}")
