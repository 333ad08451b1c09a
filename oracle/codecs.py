"""Number formats used by the oracle: OCP FP8 E4M3 and bfloat16.

TEST INFRASTRUCTURE. Part of the CPU oracle; only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it. Nothing here is
shared with the HIP library.

The pages fix only that the expert weights are stored as FP8, one byte per
parameter (peacm.com repost, section 2.1 "MoE model design"; NVIDIA blog
"How NVIDIA extreme hardware-software co-design delivered a large inference
boost for Sarvam AI's sovereign models", section "Disaggregated serving", which
says the FP8 model fits one H100). Which FP8 variant is not stated; this
oracle uses OCP E4M3 (the "FN" variant): 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits, subnormals, no infinities, NaN only for S.1111.111, largest
finite magnitude 448.

Both encoders below are written as "pick the nearest representable value,
ties to the value whose significand is even, saturate beyond the largest
finite value" -- the plain definition of round-to-nearest-even with
saturation -- not as bit tricks, so a reader can check them by eye.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def _e4m3_decode_code(code: int) -> float:
    """Value of one E4M3 byte, written out from the format's field definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:  # subnormal: 2^(1-bias) * 0.mmm
        return sign * (2.0 ** -6) * (man_field / 8.0)
    return sign * (2.0 ** (exp_field - 7)) * (1.0 + man_field / 8.0)


# Table of all 256 codes -> float64.
E4M3_TABLE = np.array([_e4m3_decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values, in code order 0x00..0x7E; value is increasing in
# the code, so the index into this array *is* the code.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_E4M3_POS) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (NaN codes give NaN)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(values: np.ndarray) -> np.ndarray:
    """Finite float values -> uint8 E4M3 codes, round-to-nearest-even, saturating.

    Magnitudes at or beyond 448 become 448 (code 0x7E). The sign bit is kept,
    so a negative value that rounds to zero becomes 0x80. Inputs are compared
    in float64, which holds every float32 exactly, so the decision made for a
    float32 input is the exact one.
    """
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    mag = np.abs(v)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")  # first table value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= E4M3_MAX, 0x7E, code)
    code = np.where(mag <= _E4M3_POS[0], 0, code)  # exact zero
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits.
# ---------------------------------------------------------------------------

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(values: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), as float64.

    Written from the definition: a normal bfloat16 has an 8-bit significand
    m * 2^(e-8) with 128 <= m < 256; the nearest such value for x = f * 2^e
    (frexp: 0.5 <= f < 1) is rint(f * 256) * 2^(e-8), and numpy's rint rounds
    halves to even. Handles the normal range only, which covers every value
    this layer produces; subnormal bfloat16 results raise.
    """
    v = np.asarray(values, dtype=np.float64)
    f, e = np.frexp(v)
    r = np.ldexp(np.rint(f * 256.0), e - 8)
    nz = v != 0
    if np.any(np.abs(v[nz]) < 2.0 ** -126):
        raise ValueError("bf16_round: subnormal result not supported")
    return r


def bf16_encode(values: np.ndarray) -> np.ndarray:
    """float64 -> uint16 bfloat16 bit patterns (round to nearest even)."""
    r = bf16_round(values).astype(np.float32)  # exact: r has 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)
