"""The QK-Norm + RoPE oracle against its pins, and planted mistakes in it
(on the CPU) that at least one pin must catch."""
import numpy as np
import pytest

from oracle import qk_rope
from tests import qk_pins


@pytest.mark.parametrize("pin", qk_pins.ALL, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _any_pin_fails():
    for pin in qk_pins.ALL:
        try:
            pin()
        except AssertionError:
            return True
    return False


ORIG = {n: getattr(qk_rope, n) for n in ["rms_norm_heads", "rope_angles", "pair_views", "rope",
                                         "qk_norm_rope"]}


def _sin_sign(x, positions, theta, style):
    return ORIG["rope"](x, -np.asarray(positions), theta, style)


def _freq_i_over_hd(positions, head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.asarray(positions, np.float64)[:, None] * np.power(theta, -i / head_dim)[None, :]


def _styles_swapped(head_dim, style):
    return ORIG["pair_views"](head_dim, "halves" if style == "interleaved" else "interleaved")


def _eps_outside_sqrt(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(w, np.float64)


def _mean_over_all_heads(x, w, eps):
    x = np.asarray(x, np.float64)
    if x.ndim < 2:
        return ORIG["rms_norm_heads"](x, w, eps)
    ms = np.mean(x * x, axis=(-2, -1), keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def _weights_swapped(qkv, positions, q_weight, k_weight, *rest):
    return ORIG["qk_norm_rope"](qkv, positions, k_weight, q_weight, *rest)


def _positions_off_by_one(qkv, positions, *rest):
    return ORIG["qk_norm_rope"](qkv, np.asarray(positions) + 1, *rest)


def _rotate_then_norm(qkv, positions, q_weight, k_weight, n_q, n_kv, head_dim, q_offset,
                      k_offset, eps, theta, style):
    out = np.array(qkv, dtype=np.float64, copy=True)
    T = out.shape[0]
    for off, nh, w in ((q_offset, n_q, q_weight), (k_offset, n_kv, k_weight)):
        cols = slice(off, off + nh * head_dim)
        heads = out[:, cols].reshape(T, nh, head_dim)
        out[:, cols] = ORIG["rms_norm_heads"](ORIG["rope"](heads, positions, theta, style), w,
                                              eps).reshape(T, -1)
    return out


MUTANTS = {
    "sin_sign_flipped": ("rope", _sin_sign),
    "frequency_exponent_i_over_hd": ("rope_angles", _freq_i_over_hd),
    "pairings_swapped": ("pair_views", _styles_swapped),
    "eps_outside_sqrt": ("rms_norm_heads", _eps_outside_sqrt),
    "norm_over_all_heads": ("rms_norm_heads", _mean_over_all_heads),
    "q_k_weights_swapped": ("qk_norm_rope", _weights_swapped),
    "positions_off_by_one": ("qk_norm_rope", _positions_off_by_one),
    "rotate_before_norm": ("qk_norm_rope", _rotate_then_norm),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(qk_rope, attr, fn)
    assert _any_pin_fails(), f"no pin catches mutant {name}"
