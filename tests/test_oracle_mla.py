"""CPU tests of the float64 MLA oracle against its pins (no GPU needed)."""
from __future__ import annotations

import inspect

import numpy as np
import pytest

import oracle
from oracle import naive_mla
from tests import oracle_mla_pins as pins

NAMES = ("mla_naive", "mla_absorbed", "mla_absorb_q", "mla_latent_attention", "mla_up_project")


class _Ora:
    attention_forward = staticmethod(oracle.attention_forward)


for _n in NAMES:
    setattr(_Ora, _n, staticmethod(getattr(naive_mla, _n)))


@pytest.mark.parametrize("pin", pins.PINS_MLA, ids=lambda f: f.__name__)
def test_mla_pin(pin):
    pin(_Ora)


MUTATIONS = {
    "mask_direction": ("return j > s + (T - S_)", "return j < s + (T - S_)"),
    "mask_top_left": ("return j > s + (T - S_)", "return j > s"),
    "rope_dropped_naive": ("K = np.concatenate([c_kv[b] @ W_uk[h].T, k_pe[b]], axis=1)",
                           "K = np.concatenate([c_kv[b] @ W_uk[h].T, 0 * k_pe[b]], axis=1)"),
    "absorb_wrong_contraction": ('np.einsum("bhsd,hdc->bhsc", q_nope, W_uk)',
                                 'np.einsum("bhsd,hdc->bhsc", q_nope, W_uk[::-1])'),
    "latent_values_from_rope_end": ("out[b, h] = P @ kv[b, :, :d_c]", "out[b, h] = P @ kv[b, :, -d_c:]"),
    "up_project_transposed_heads": ('np.einsum("bhsc,hvc->bhsv", out_lat, W_uv)',
                                    'np.einsum("bhsc,hvc->bhsv", out_lat, W_uv[::-1])'),
    "lse_without_max": ("return E / l[:, None], m + np.log(l)", "return E / l[:, None], np.log(l)"),
    "scale_dropped_latent": ("X = sm_scale * (q_lat[b, h] @ kv[b].T)", "X = (q_lat[b, h] @ kv[b].T)"),
}


def _mutant(old, new):
    src = inspect.getsource(naive_mla)
    assert old in src, f"mutation target not found: {old!r}"
    ns = {"__name__": "mla_mutant"}
    exec(compile(src.replace(old, new), "<mla_mutant>", "exec"), ns)

    class M:
        attention_forward = staticmethod(oracle.attention_forward)
    for n in NAMES:
        setattr(M, n, staticmethod(ns[n]))
    return M


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mla_pins_catch_mutant(name):
    m = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.PINS_MLA:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
