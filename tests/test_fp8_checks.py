"""CPU checks of the FP8-decision validator used by the GPU tests: it accepts
neighbouring codes caused by small perturbations of h and rejects anything
else."""
import numpy as np
import pytest

from oracle import codecs
from oracle import moe as omoe
from tests import fp8_checks as FC


def _h(seed=0, R=40, F=256):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((R, F)) * 2
    u = rng.standard_normal((R, F)) * 2
    return omoe.silu(g) * u


def test_accepts_perturbed_decisions():
    h = _h(R=400)
    hp = h * (1 + np.random.default_rng(1).uniform(-1e-4, 1e-4, h.shape))
    q, s = omoe.quantize_blocks_e4m3(hp)
    flips, dhq = FC.validate_h(h, q, s)
    assert flips > 0  # the perturbation does move some codes
    assert np.abs(dhq).max() > 0


def test_exact_decisions_have_no_flips():
    h = _h(2)
    q, s = omoe.quantize_blocks_e4m3(h)
    flips, dhq = FC.validate_h(h, q, s)
    assert flips == 0 and np.all(dhq == 0)


def test_rejects_a_wrong_code():
    h = _h(3)
    q, s = omoe.quantize_blocks_e4m3(h)
    q = q.copy()
    # move a mid-range code two steps away
    i = np.argwhere((q & 0x7F) > 0x20)[5]
    q[tuple(i)] = q[tuple(i)] + 2
    with pytest.raises(AssertionError):
        FC.validate_h(h, q, s)


def test_rejects_a_sign_error_and_a_bad_scale():
    h = _h(4)
    q, s = omoe.quantize_blocks_e4m3(h)
    q2 = q.copy()
    i = np.argwhere((q & 0x7F) > 0x30)[0]
    q2[tuple(i)] ^= 0x80
    with pytest.raises(AssertionError):
        FC.validate_h(h, q2, s)
    with pytest.raises(AssertionError):
        FC.validate_h(h, q, s * np.float32(1.01))


def test_down_effect_bounds_the_output_change():
    rng = np.random.default_rng(5)
    R, F, d = 6, 256, 64
    h = _h(6, R, F)
    q, s = omoe.quantize_blocks_e4m3(h)
    hp = h * (1 + rng.uniform(-5e-5, 5e-5, h.shape))
    q2, s2 = omoe.quantize_blocks_e4m3(hp)
    ew = omoe.ExpertWeights(None, None, codecs.e4m3_encode(rng.standard_normal((d, F)) * 50),
                            np.full(d, 0.01, np.float32))
    _, dhq = FC.validate_h(h, q2, s2)
    diff = np.abs(omoe.down_fp8(q2, s2, ew) - omoe.down_fp8(q, s, ew))
    assert np.all(diff <= FC.down_effect(dhq, ew) * (1 + 1e-9) + 1e-12)
