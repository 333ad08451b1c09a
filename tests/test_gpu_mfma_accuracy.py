"""How exactly gfx950's FP8 matrix-core instruction sums its products, measured
on the device. The FP8 parity checks (tests/fp8_checks.py) bound the error of
one v_mfma_f32_16x16x128_f8f6f4 by MFMA_EPS times the sum of its |a*b|; this
test measures that error on operands distributed like the layer's (per-row
quantised normal rows of x codes against per-row quantised normal weight rows)
and asserts the bound there, and records two further figures: the error on
codes drawn uniformly over all finite E4M3 values (a wider dynamic range
inside each product group), and the structure of the loss (one product of 1
beside 127 products of 2^-t). Expected values are exact float64 sums of
exactly decoded E4M3 products."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from oracle import codecs
from tests import gpu_helpers as H
from tests.fp8_checks import MFMA_EPS

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_fp8_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        raise ImportError(f"{PROBE} is missing: build with `python -m mixture_experts_softmax_amd.build`")
    L = C.CDLL(PROBE)
    L.mfma_fp8_probe.restype = C.c_int
    L.mfma_fp8_probe.argtypes = [C.c_void_p] * 3 + [C.c_int, C.c_void_p]
    return L


def run_mfma(a: np.ndarray, b: np.ndarray):
    """a, b: uint8 [n][64][32] operand bytes per lane. Returns the GPU's
    D [n][16][16] and the exact D and sum |a*b| (float64)."""
    n = a.shape[0]
    assert a.shape == b.shape == (n, 64, 32) and a.dtype == b.dtype == np.uint8
    da, db = torch.from_numpy(a).to(H.DEV), torch.from_numpy(b).to(H.DEV)
    out = torch.empty((n, 64, 4), dtype=torch.float32, device=H.DEV)
    st = _probe().mfma_fp8_probe(da.data_ptr(), db.data_ptr(), out.data_ptr(), n,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"launch failed: {st}"
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    lane = np.arange(64)
    D = np.empty((n, 16, 16))
    for q in range(4):
        D[:, 4 * (lane // 16) + q, lane % 16] = o[:, :, q]
    av = codecs.e4m3_decode(a).reshape(n, 4, 16, 32)  # (group, row, byte)
    bv = codecs.e4m3_decode(b).reshape(n, 4, 16, 32)  # (group, column, byte)
    exact = np.einsum("ngrp,ngcp->nrc", av, bv)
    absum = np.einsum("ngrp,ngcp->nrc", np.abs(av), np.abs(bv))
    return D, exact, absum


def _quantised_normal_rows(rng, n):
    """Per-lane rows of E4M3 codes of N(0, 1) values scaled so the lane's
    amax is 448 (as the kernels' x and weight rows are)."""
    v = rng.standard_normal((n, 64, 32))
    v = v / np.abs(v).max(axis=2, keepdims=True) * 448.0
    return codecs.e4m3_encode(v.astype(np.float32))


def test_mfma_fp8_error_within_parity_bound():
    rng = np.random.default_rng(2024)
    D, exact, absum = run_mfma(_quantised_normal_rows(rng, 4000), _quantised_normal_rows(rng, 4000))
    rel = np.abs(D - exact) / absum
    H.say(f"  layer-like operands, {rel.size} sums of 128 products: error / sum|ab| "
          f"max {rel.max():.3e} mean {rel.mean():.3e} p99.9 {np.quantile(rel, 0.999):.3e}; "
          f"bound MFMA_EPS = 2^-15 = {MFMA_EPS:.3e} ({MFMA_EPS / rel.max():.1f}x the largest)")
    assert rel.max() <= MFMA_EPS
    # uniform over all finite codes: recorded, not bounded by MFMA_EPS
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a = finite[rng.integers(0, finite.size, (4000, 64, 32))]
    b = finite[rng.integers(0, finite.size, (4000, 64, 32))]
    D, exact, absum = run_mfma(a, b)
    ok = absum > 0
    rel = np.abs(D - exact)[ok] / absum[ok]
    H.say(f"  uniform finite codes: error / sum|ab| max {rel.max():.3e} mean {rel.mean():.3e}")
    assert np.all(np.isfinite(D))


def test_mfma_fp8_loss_structure():
    """One product 1 * 1 at lane group 0, byte 0 of row 0 / column 0, and 127
    products of +2^-t (t = 1..18) at every other position: how many of the
    small products the sum loses."""
    rows = []
    for t in range(1, 19):
        a = np.zeros((1, 64, 32), np.uint8)
        b = np.zeros((1, 64, 32), np.uint8)
        one = codecs.e4m3_encode(np.float32(1.0))
        ta, tb = (t + 1) // 2, t // 2
        a[0, [0, 16, 32, 48], :] = codecs.e4m3_encode(np.float32(2.0 ** -ta))
        b[0, [0, 16, 32, 48], :] = codecs.e4m3_encode(np.float32(2.0 ** -tb))
        a[0, 0, 0] = one
        b[0, 0, 0] = one
        D, exact, _ = run_mfma(a, b)
        lost = (exact[0, 0, 0] - D[0, 0, 0]) / 2.0 ** -t
        rows.append((t, lost))
        assert abs(exact[0, 0, 0] - (1 + 127 * 2.0 ** -t)) < 1e-15
    H.say("  1 + 127 x 2^-t: products lost per t: " + ", ".join(f"t={t}: {l:g}" for t, l in rows))
    # small products far enough below the large one vanish, but never more
    # than the seven that share its group of eight
    assert all(-7 <= l <= 7 for _, l in rows)
