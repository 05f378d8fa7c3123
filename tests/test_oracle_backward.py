"""CPU tests of the float64 backward oracle against its pins (no GPU needed)."""
from __future__ import annotations

import inspect

import numpy as np
import pytest

import oracle
from oracle import naive_backward
from tests import oracle_backward_pins as pins


class _Ora:
    attention_forward = staticmethod(oracle.attention_forward)
    attention_backward = staticmethod(oracle.attention_backward)
    backward_rows = staticmethod(oracle.backward_rows)
    backward_keys = staticmethod(oracle.backward_keys)


@pytest.mark.parametrize("pin", pins.PINS_BWD, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(_Ora)


def test_rows_and_keys_match_full():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 600, 8))
    k = rng.standard_normal((1, 2, 700, 8))
    v = rng.standard_normal((1, 2, 700, 8))
    dO = rng.standard_normal((1, 4, 600, 8))
    for causal in (False, True):
        dQ, dK, dV = oracle.attention_backward(q, k, v, dO, is_causal=causal, sm_scale=0.3)
        rows = np.array([0, 1, 511, 512, 599])
        np.testing.assert_allclose(
            oracle.backward_rows(q, k, v, dO, 0, 3, rows, is_causal=causal, sm_scale=0.3),
            dQ[0, 3, rows], rtol=0, atol=1e-12)
        keys = np.array([0, 99, 100, 699])
        bk, bv = oracle.backward_keys(q, k, v, dO, 0, 1, keys, is_causal=causal, sm_scale=0.3)
        np.testing.assert_allclose(bk, dK[0, 1, keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(bv, dV[0, 1, keys], rtol=0, atol=1e-12)


# Each mutant plants one plausible mistake in a copy of the backward oracle's
# source (every occurrence of the target text); at least one pin must fail.
MUTATIONS = {
    "softmax_grad_without_rowsum": ("(dP - Dl[:, None])", "dP"),
    "rowsum_without_o": ("Dl = (dO * O).sum(axis=1)", "Dl = dO.sum(axis=1)"),
    "dq_scale_dropped": ("= sm_scale * (dS @ k[b, g])", "= (dS @ k[b, g])"),
    "dk_not_summed_over_group": ("dK[b, g] += sm_scale", "dK[b, g] = sm_scale"),
    "dv_not_summed_over_group": ("dV[b, g] += P.T @ dO", "dV[b, g] = P.T @ dO"),
    "dk_from_p": ("sm_scale * (dS.T @ q[b, h])", "sm_scale * (P.T @ q[b, h])"),
    "mask_excludes_diagonal": ("> rows[:, None] + off", ">= rows[:, None] + off"),
    "causal_offset_ignored": ("off = N_kv - N_q if is_causal else 0", "off = 0"),
    "keys_softmax_grad_without_rowsum": ("dSk = Pk * (dPk - Dl[:, None])", "dSk = Pk * dPk"),
    "keys_dv_scaled": ("dV += Pk.T @ dO", "dV += sm_scale * (Pk.T @ dO)"),
    "dv_scaled": ("dV[b, g] += P.T @ dO", "dV[b, g] += sm_scale * (P.T @ dO)"),
    "head_map_modulo": ("g = kv_head(h, H_q, H_kv)", "g = h % H_kv"),
    "keys_row_subset_ignored": ("rows = np.arange(N_q) if rows is None else np.asarray(rows, dtype=np.int64)",
                                "rows = np.arange(N_q)"),
    "keys_row_blocks_skip_first": ("r = rows[s:s + ROW_BLOCK]", "r = rows[s + 1:s + ROW_BLOCK]"),
    "supplied_output_ignored": ("O = P @ v[b, g] if out is None else out[b, h]", "O = P @ v[b, g]"),
}


def _mutant(old, new):
    src = inspect.getsource(naive_backward)
    assert old in src, f"mutation target not found: {old!r}"
    src = src.replace("from .naive_attention import", "from oracle.naive_attention import")
    ns = {"__name__": "backward_mutant"}
    exec(compile(src.replace(old, new), "<backward_mutant>", "exec"), ns)

    class M:
        attention_forward = staticmethod(oracle.attention_forward)
        attention_backward = staticmethod(ns["attention_backward"])
        backward_rows = staticmethod(ns["backward_rows"])
        backward_keys = staticmethod(ns["backward_keys"])
    return M


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_pins_catch_mutant(name):
    m = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.PINS_BWD:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
