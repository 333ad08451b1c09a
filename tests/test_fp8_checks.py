"""CPU checks of the FP8-decision validator used by the GPU tests: it accepts
neighbouring codes caused by perturbations of g and u within the MFMA error
bound, and rejects wrong codes, wrong signs and wrong scales."""
import numpy as np
import pytest

from oracle import codecs
from oracle import moe as omoe
from tests import fp8_checks as FC


def _expert(seed, R=64, d=512, F=256):
    rng = np.random.default_rng(seed)
    xq, sx = omoe.quantize_rows_e4m3(rng.standard_normal((R, d)))
    w13 = codecs.e4m3_encode(rng.standard_normal((2 * F, d)) * 100)
    s13 = np.full(2 * F, 1.0 / (100 * np.sqrt(d)), np.float32)
    w2 = codecs.e4m3_encode(rng.standard_normal((d, F)) * 100)
    ew = omoe.ExpertWeights(w13, s13, w2, np.full(d, 1.0 / (100 * np.sqrt(F)), np.float32))
    return xq, sx, ew


def _kernel_like(xq, sx, ew, seed, frac):
    """h from g, u perturbed by up to frac of the MFMA error bound."""
    F = ew.w13.shape[0] // 2
    gu = omoe.gate_up_fp8(xq, sx, ew)
    absum = np.abs(codecs.e4m3_decode(xq)) @ np.abs(codecs.e4m3_decode(ew.w13)).T
    absum *= sx[:, None] * ew.w13_scale[None, :]
    gu = gu + np.random.default_rng(seed).uniform(-1, 1, gu.shape) * frac * FC.MFMA_EPS * absum
    return omoe.silu(gu[:, :F]) * gu[:, F:]


def test_accepts_decisions_within_the_bound():
    xq, sx, ew = _expert(0, R=256)
    q, s = omoe.quantize_blocks_e4m3(_kernel_like(xq, sx, ew, 1, 0.25))
    flips, dhq = FC.validate_h(xq, sx, ew, q, s)
    assert flips > 0  # the perturbation does move some codes
    assert np.abs(dhq).max() > 0


def test_exact_decisions_have_no_flips():
    xq, sx, ew = _expert(2)
    q, s = omoe.quantize_blocks_e4m3(omoe.swiglu_h_fp8(xq, sx, ew))
    flips, dhq = FC.validate_h(xq, sx, ew, q, s)
    assert flips == 0 and np.all(dhq == 0)


def test_rejects_a_wrong_code():
    xq, sx, ew = _expert(3)
    q, s = omoe.quantize_blocks_e4m3(omoe.swiglu_h_fp8(xq, sx, ew))
    q = q.copy()
    i = tuple(np.argwhere((q & 0x7F) > 0x40)[5])
    q[i] = q[i] + 2
    with pytest.raises(AssertionError):
        FC.validate_h(xq, sx, ew, q, s)


def test_rejects_a_sign_error_and_a_bad_scale():
    xq, sx, ew = _expert(4)
    q, s = omoe.quantize_blocks_e4m3(omoe.swiglu_h_fp8(xq, sx, ew))
    q2 = q.copy()
    i = tuple(np.argwhere((q & 0x7F) > 0x40)[0])
    q2[i] ^= 0x80
    with pytest.raises(AssertionError):
        FC.validate_h(xq, sx, ew, q2, s)
    with pytest.raises(AssertionError):
        FC.validate_h(xq, sx, ew, q, s * np.float32(1.01))


def test_down_effect_bounds_the_output_change():
    xq, sx, ew = _expert(6, R=32)
    q, s = omoe.quantize_blocks_e4m3(omoe.swiglu_h_fp8(xq, sx, ew))
    q2, s2 = omoe.quantize_blocks_e4m3(_kernel_like(xq, sx, ew, 7, 0.25))
    _, dhq = FC.validate_h(xq, sx, ew, q2, s2)
    diff = np.abs(omoe.down_fp8(q2, s2, ew) - omoe.down_fp8(q, s, ew))
    assert np.all(diff <= FC.down_effect(dhq, ew) * (1 + 1e-9) + 1e-12)


def test_flip_rate_cap_is_over_the_whole_call():
    FC.check_flip_rate(11, 1000)      # 1% of 1000 codes (+1)
    with pytest.raises(AssertionError):
        FC.check_flip_rate(12, 1000)
    FC.check_flip_rate(1, 50)         # one decision in a tiny call is allowed
