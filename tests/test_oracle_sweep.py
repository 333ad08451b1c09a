"""The oracle's whole layer against the scalar brute-force loop (every
expert run on every token, masked by the top-k selection) on the tiny
float32 workload and on a seeded sweep of small random shapes: T <= 4,
E <= 6, k <= E, d and F in {128, 256}, with and without a shared expert or
router bias, FP8 and float32 weights. CPU only."""
import math

import numpy as np
import pytest

from oracle import brute, codecs
from oracle import inputs as oinputs
from oracle import moe
from synthetic import CONFIGS, make_layer
from tests import oracle_pins as P


def _tuples(ew, fp8):
    return (ew.w13, ew.w13_scale if fp8 else None, ew.w2, ew.w2_scale if fp8 else None)


def test_tiny_workload_vs_brute():
    cfg = CONFIGS["tiny"]
    lt = make_layer(cfg, device="cpu", hooks=oinputs.HOOKS)
    inp = oinputs.layer_inputs(lt)
    ref = moe.layer_forward(inp)
    experts = [_tuples(inp.expert(e), False) for e in range(cfg.E)]
    shared = _tuples(inp.shared, False) if inp.shared is not None else None
    ids, w, y = brute.brute_layer(moe.activations(inp), moe.router_weight(inp), inp.router_bias,
                                  cfg.k, experts, shared, fp8=False)
    assert np.array_equal(ref.ids, ids)
    assert np.allclose(ref.w, w, atol=1e-14, rtol=0)
    assert np.allclose(ref.y64, y, atol=1e-10, rtol=0)


def _random_f32_layer(rng, T, d, E, k, F, Fs, bias):
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None

    def mk(F_):
        return moe.ExpertWeights((rng.standard_normal((2 * F_, d)) / math.sqrt(d)).astype(np.float32),
                                 None,
                                 (rng.standard_normal((d, F_)) / math.sqrt(F_)).astype(np.float32),
                                 None)
    experts = [mk(F) for _ in range(E)]
    shared = mk(Fs) if Fs else None
    return moe.LayerInputs("f32", x, wr, b, k, E, lambda e: experts[e], shared), experts, shared


@pytest.mark.parametrize("seed", range(8))
def test_random_sweep_vs_brute(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 5))
    E = int(rng.integers(1, 7))
    k = int(rng.integers(1, E + 1))
    d = int(rng.choice([128, 256]))
    F = int(rng.choice([128, 256]))
    Fs = int(rng.choice([0, 128]))
    bias = bool(rng.integers(0, 2))
    fp8 = seed % 2 == 0
    if fp8:
        inp, experts, shared = P._random_fp8_layer(2000 + seed, T, d, E, k, F, Fs, bias=bias)
        x = codecs.bf16_decode(inp.x)
        wr = codecs.bf16_decode(inp.w_router)
    else:
        inp, experts, shared = _random_f32_layer(rng, T, d, E, k, F, Fs, bias)
        x, wr = inp.x.astype(np.float64), inp.w_router.astype(np.float64)
    ref = moe.layer_forward(inp)
    ids, w, y = brute.brute_layer(x, wr, inp.router_bias, k, [_tuples(e, fp8) for e in experts],
                                  _tuples(shared, fp8) if shared is not None else None, fp8=fp8)
    assert np.array_equal(ref.ids, ids), (T, E, k, d, F, Fs, bias, fp8)
    assert np.allclose(ref.w, w, atol=1e-14, rtol=0)
    assert np.allclose(ref.y64, y, atol=1e-9, rtol=0)
