"""GPU test of attn_fwd_splitkv_static, the split forward that allocates
nothing (its key-split partials live in the library's static device scratch).

Called through the C ABI (ctypes binding) and compared with attn_fwd_splitkv
on the same inputs with the same split count, which runs the same kernels on
a caller workspace: the outputs must be bit-identical.  Two calls in a row
(the second smaller, so it reuses scratch the first left behind), then the
library's own split choice, the rejection of an explicit split count whose
partials exceed the scratch, and a check against the float64 oracle.
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


def _pair(ea, B, H_q, H_kv, N_q, N_kv, D, causal, n_splits, seed):
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in workloads.make_inputs(B, H_q, H_kv, N_q, D, seed, N_kv=N_kv))
    ref_o = torch.full((B, H_q, N_q, D), float("nan"), dtype=torch.bfloat16, device=dev)
    ref_l = torch.full((B, H_q, N_q), float("nan"), dtype=torch.float32, device=dev)
    ns = n_splits if n_splits > 0 else ea.attn_splitkv_num_splits(B, H_q, H_kv, N_q, N_kv, D, causal)
    nbytes = ea.attn_splitkv_workspace_size(B, H_q, N_q, D, ns)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    ea.attn_fwd_splitkv(q, k, v, ref_o, ref_l, is_causal=causal, n_splits=ns, workspace=ws)
    o = torch.full_like(ref_o, float("nan"))
    l = torch.full_like(ref_l, float("nan"))
    ea.attn_fwd_splitkv_static(q, k, v, o, l, is_causal=causal, n_splits=n_splits)
    torch.cuda.synchronize()
    return (q, k, v), (o.cpu(), l.cpu()), (ref_o.cpu(), ref_l.cpu()), ns


def _same(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and \
        torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_static_scratch_matches_workspace_entry_point_twice(ea):
    # a decode step against a long cache (many splits), then a smaller problem
    for shape in [(1, 32, 8, 1, 65536, 128, True, 64), (1, 8, 2, 37, 3000, 64, False, 5)]:
        B, H_q, H_kv, N_q, N_kv, D, causal, ns = shape
        assert ea.attn_splitkv_workspace_size(B, H_q, N_q, D, ns) <= ea.attn_static_scratch_bytes()
        _, got, ref, _ = _pair(ea, B, H_q, H_kv, N_q, N_kv, D, causal, ns, seed=7700 + N_q)
        assert torch.isfinite(got[0].float()).all() and torch.isfinite(got[1]).all()
        assert _same(got, ref), f"static-scratch output differs from the workspace call at {shape}"


def test_static_scratch_library_split_choice(ea):
    B, H_q, H_kv, N_q, N_kv, D, causal = 1, 32, 32, 1, 16384, 128, True
    (q, k, v), got, ref, ns = _pair(ea, B, H_q, H_kv, N_q, N_kv, D, causal, 0, seed=7800)
    assert ns > 1
    assert _same(got, ref)
    O_ref, L_ref = oracle.attention_forward(*(workloads.to_float64(x.cpu()) for x in (q, k, v)),
                                            is_causal=causal, sm_scale=1.0 / math.sqrt(D))
    o = got[0].double().numpy()
    assert np.all(np.abs(o - O_ref) <= 2e-2 + 2e-2 * np.abs(O_ref))
    assert np.all(np.abs(got[1].double().numpy() - L_ref) <= 1e-3)


def test_static_scratch_rejects_oversized_split_request(ea):
    dev = torch.device("cuda", 0)
    B, H_q, H_kv, N_q, N_kv, D = 1, 64, 8, 128, 4096, 128
    ns = 64
    assert ea.attn_splitkv_workspace_size(B, H_q, N_q, D, ns) > ea.attn_static_scratch_bytes()
    q = torch.zeros((B, H_q, N_q, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, H_kv, N_kv, D), dtype=torch.bfloat16, device=dev)
    o = torch.full_like(q, 3.0)
    l = torch.full((B, H_q, N_q), 5.0, dtype=torch.float32, device=dev)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_fwd_splitkv_static(q, k, k, o, l, n_splits=ns)
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(l == 5.0)
    # the library's own choice is lowered to fit and runs
    ea.attn_fwd_splitkv_static(q, k, k, o, l, n_splits=0)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.allclose(l, torch.full_like(l, math.log(N_kv)))
