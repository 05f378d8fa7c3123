"""CPU tests of the float64 oracle against its pins (no GPU needed)."""
from __future__ import annotations

import inspect
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import naive_attention
import workloads
from tests import blockwise_reference, oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_bf16_upcast_is_exact():
    q, _, _ = workloads.make_inputs(1, 2, 1, 64, 32, seed=7)
    x64 = workloads.to_float64(q)
    back = torch.from_numpy(x64).to(torch.bfloat16)
    assert torch.equal(back.view(torch.int16), q.view(torch.int16))


def test_workload_generation_is_deterministic():
    a = workloads.make_inputs(1, 2, 1, 8, 16, seed=3)
    b = workloads.make_inputs(1, 2, 1, 8, 16, seed=3)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = workloads.make_inputs(1, 2, 1, 8, 16, seed=4)
    assert not torch.equal(a[0], c[0])


@pytest.mark.parametrize("tile", [(1, 1), (3, 7), (7, 3), (16, 16), (70, 70)])
@pytest.mark.parametrize("l_init", [0.0, 1.0])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_recurrence_equals_naive(tile, l_init, causal):
    rng = np.random.default_rng(17)
    B, H_q, H_kv, N, D = 2, 4, 2, 70, 16
    q = rng.standard_normal((B, H_q, N, D))
    k = rng.standard_normal((B, H_kv, N, D))
    v = rng.standard_normal((B, H_kv, N, D))
    O, L = oracle.attention_forward(q, k, v, is_causal=causal, sm_scale=0.25)
    Ob, Lb = blockwise_reference.blockwise_attention(
        q, k, v, is_causal=causal, sm_scale=0.25, tile_m=tile[0], tile_n=tile[1], l_init=l_init)
    np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-12)


def test_rows_api_matches_full():
    q, k, v = (workloads.to_float64(t) for t in workloads.make_inputs(1, 4, 2, 300, 8, seed=9))
    O, L = oracle.attention_forward(q, k, v, is_causal=True, sm_scale=0.3)
    rows = np.array([0, 1, 150, 299, 7])
    Or, Lr = oracle.attention_rows(q, k, v, 0, 3, rows, is_causal=True, sm_scale=0.3)
    np.testing.assert_allclose(Or, O[0, 3, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lr, L[0, 3, rows], rtol=0, atol=1e-13)


def test_row_blocks_span_several_blocks():
    """More rows than one oracle row block: blocks must not change any value."""
    q, k, v = (workloads.to_float64(t) for t in workloads.make_inputs(1, 1, 1, 1100, 4, seed=8))
    O, L = oracle.attention_forward(q, k, v, is_causal=True, sm_scale=0.5)
    rows = np.arange(1100)
    for i in (0, 511, 512, 513, 1023, 1024, 1099):
        Oi, Li = oracle.attention_rows(q, k, v, 0, 0, rows[i:i + 1], is_causal=True, sm_scale=0.5)
        np.testing.assert_allclose(Oi[0], O[0, 0, i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Li[0], L[0, 0, i], rtol=0, atol=1e-13)


def test_golden_regression():
    """Stored oracle output (written by tests/golden/make_golden.py) is unchanged."""
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        q, k, v = (workloads.to_float64(t) for t in workloads.make_inputs(
            case["B"], case["H_q"], case["H_kv"], case["N"], case["D"], case["seed"]))
        O, L = oracle.attention_forward(q, k, v, is_causal=case["causal"],
                                        sm_scale=case["sm_scale"])
        np.testing.assert_allclose(O.ravel(), np.array(case["O"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L.ravel(), np.array(case["LSE"]), rtol=0, atol=1e-13)


# ------------------------------------------------------------------ mutations
# Each mutant plants one plausible mistake in a copy of the oracle's source; at
# least one pin must catch it.  The first three are the mistakes the page
# "Triton Cuda Attention" lists under "常见错误" (modulo head map, missing final
# division by l) plus their neighbours.
MUTATIONS = {
    "modulo_head_map": ("(h * H_kv) // H_q", "h % H_kv"),
    "missing_div_l": ("out[s:s + ROW_BLOCK] = (E @ Vg) / l[:, None]",
                      "out[s:s + ROW_BLOCK] = (E @ Vg)"),
    "no_max_subtraction": ("np.exp(S - m[:, None])", "np.exp(S)"),
    "exp_sign_flipped": ("np.exp(S - m[:, None])", "np.exp(m[:, None] - S)"),
    "mask_direction": ("j > r[:, None]", "j < r[:, None]"),
    "mask_excludes_diagonal": ("j > r[:, None]", "j >= r[:, None]"),
    "lse_without_max": ("lse[s:s + ROW_BLOCK] = m + np.log(l)",
                        "lse[s:s + ROW_BLOCK] = np.log(l)"),
    "scale_dropped": ("S = sm_scale * (", "S = ("),
    "causal_key_range_short": ("nk = int(r.max()) + off + 1 if is_causal else N_kv",
                               "nk = int(r.max()) + off if is_causal else N_kv"),
    "causal_offset_ignored": ("off = N_kv - N_q if is_causal else 0", "off = 0"),
    "causal_offset_wrong_sign": ("off = N_kv - N_q if is_causal else 0",
                                 "off = N_q - N_kv if is_causal else 0"),
    "v_replaced_by_k": ("Vg = v[b, g, :nk, :]", "Vg = k[b, g, :nk, :]"),
    "keys_reversed": ("Kg = k[b, g, :nk, :]", "Kg = k[b, g, :nk, :][::-1]"),
    "merge_without_max": ("w = np.exp(lse_parts - m[None])", "w = np.exp(lse_parts)"),
    "merge_lse_without_max": ("lse = m + np.log(tot)", "lse = np.log(tot)"),
    "merge_unnormalised": ("(w[..., None] * o_parts).sum(axis=0) / tot[..., None]",
                           "(w[..., None] * o_parts).sum(axis=0)"),
}


def _mutant(old, new):
    src = inspect.getsource(naive_attention)
    assert old in src, f"mutation target not found: {old!r}"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "<oracle_mutant>", "exec"), ns)

    class M:
        pass
    m = M()
    for name in ("attention_forward", "attention_rows", "kv_head", "merge_partials"):
        setattr(m, name, ns[name])
    return m


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutant(name):
    m = _mutant(*MUTATIONS[name])
    caught = []
    for pin in oracle_pins.PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"


def test_blockwise_missing_rescale_is_caught():
    """Dropping acc*alpha from the recurrence (a listed common mistake) must
    disagree with the naive oracle."""
    src = inspect.getsource(blockwise_reference)
    old = "acc = alpha[:, None] * acc + p @ v[b, g, cols]"
    assert old in src
    ns = {"__name__": "blockwise_mutant"}
    exec(compile(src.replace(old, "acc = acc + p @ v[b, g, cols]"), "<m>", "exec"), ns)
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(3))
    O, _ = oracle.attention_forward(q, k, v, is_causal=True, sm_scale=1.0)
    Ob, _ = ns["blockwise_attention"](q, k, v, is_causal=True, sm_scale=1.0, tile_m=8, tile_n=8)
    assert np.max(np.abs(Ob - O)) > 1e-3
