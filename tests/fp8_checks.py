"""Checking FP8 quantisation decisions that the GPU takes on values carrying
the FP8 matrix-core accumulation error.

gfx950's v_mfma_f32_16x16x128_f8f6f4 does not sum its 128 products exactly:
products are added in groups of 8 aligned to the group's largest product, and
bits more than 13 binary places below it are dropped (probe: one 1.0 product
with 127 products of +-2^-t loses exactly the 7 small products of its group
for every t >= 14). On normally distributed data the gate/up values h then
differ from their exact values by ~6e-5 relative (typical), so an h value that
lies that close to an E4M3 rounding midpoint can take either neighbouring
code; both are valid quantisations of h. The kernel's h, its codes and block
scales, are therefore checked like this:

  * every block scale is within H_EPS (relative) of the oracle's amax/448;
  * every code is the round-to-nearest-even code of some value within
    H_EPS (relative) of the exact h on the kernel's own block scale, i.e. it
    equals the oracle's code, or is the neighbouring code of an h that lies
    within H_EPS of the midpoint between the two;
  * such neighbouring-code decisions are rare (FLIP_MAX of all codes).

Downstream, a validated neighbouring code changes one expert output by
exactly |dh_n| * |W2[m][n]| through the down projection; the output
tolerance adds these terms and nothing else. The expected values themselves
are the oracle's alone.
"""
from __future__ import annotations

import numpy as np

from oracle import codecs
from oracle import moe as omoe

H_EPS = 2.0 ** -10    # 1e-3: ~15x the typical measured relative error of h
FLIP_MAX = 0.01       # at most 1% of h codes may take the neighbouring value


def _code_mag(v):
    return codecs.e4m3_encode(np.abs(v)) & 0x7F


def validate_h(h64: np.ndarray, q_gpu: np.ndarray, s_gpu: np.ndarray):
    """h64: exact h [R][F] (oracle); q_gpu [R][F] uint8, s_gpu [R][F/128]: the
    kernel's codes and scales. Returns (n_flips, dhq) where dhq [R][F] is the
    kernel's dequantised h minus the oracle's. Raises AssertionError when a
    decision is not a valid quantisation of h."""
    R, F = h64.shape
    nb = F // omoe.H_BLOCK
    q_ref, s_ref = omoe.quantize_blocks_e4m3(h64)
    s_ref = s_ref.reshape(R, nb)
    s_gpu = np.asarray(s_gpu, np.float32).reshape(R, nb)
    rel = np.abs(s_gpu.astype(np.float64) / s_ref.astype(np.float64) - 1.0)
    assert np.all(rel <= H_EPS), f"h block scales off by up to {rel.max():.3e}"
    # the exact h on the kernel's scale grid, and the codes reachable within H_EPS
    v = (np.asarray(h64, np.float32).reshape(R, nb, omoe.H_BLOCK)
         / s_gpu[:, :, None]).reshape(R, F).astype(np.float64)
    lo = _code_mag(v * (1.0 - H_EPS))
    hi = _code_mag(v * (1.0 + H_EPS))
    qm = q_gpu & 0x7F
    ok_mag = (qm >= np.minimum(lo, hi)) & (qm <= np.maximum(lo, hi))
    ok_sign = (qm == 0) | ((q_gpu >> 7).astype(bool) == np.signbit(v))
    bad = ~(ok_mag & ok_sign)
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"h code {q_gpu[r, c]:#x} at ({r}, {c}) is not a quantisation of "
                             f"h={h64[r, c]!r} (v={v[r, c]!r}, allowed {lo[r, c]:#x}..{hi[r, c]:#x})")
    flips = int((q_gpu != q_ref).sum())
    assert flips <= FLIP_MAX * q_gpu.size + 1, f"{flips} of {q_gpu.size} h codes differ"
    hq_gpu = codecs.e4m3_decode(q_gpu) * np.repeat(s_gpu.astype(np.float64), omoe.H_BLOCK, axis=1)
    hq_ref = codecs.e4m3_decode(q_ref) * np.repeat(s_ref.astype(np.float64), omoe.H_BLOCK, axis=1)
    return flips, hq_gpu - hq_ref


def down_effect(dhq: np.ndarray, ew: omoe.ExpertWeights) -> np.ndarray:
    """Largest change of each expert output the h differences can cause:
    |dhq| @ |W2 dequantised|^T, [R][d]."""
    w2 = np.abs(codecs.e4m3_decode(ew.w2) * np.asarray(ew.w2_scale, np.float64)[:, None])
    return np.abs(dhq) @ w2.T
