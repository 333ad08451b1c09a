"""Number formats used by the oracle: OCP FP8 E4M3, bfloat16, and the OCP
Microscaling MXFP4 weight format (E2M1 elements with one E8M0 scale per 32).

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


# ---------------------------------------------------------------------------
# MXFP4 (OCP Microscaling Formats, version 1.0): blocks of 32 FP4 E2M1
# elements sharing one E8M0 scale. Used for expert weights only.
#   E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, subnormals,
#         no infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
#   E8M0: an unsigned exponent byte e, value 2^(e - 127); 0xFF is NaN.
# Storage convention of this layer (not fixed by the spec): two elements per
# byte along the reduction dimension, element 2i in the low nibble of byte i;
# scales one byte per (row, 32-element block) in block order.
# ---------------------------------------------------------------------------

def _e2m1_decode_code(code: int) -> float:
    """Value of one E2M1 nibble, from the format's field definition."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 0x3
    man_field = code & 0x1
    if exp_field == 0:  # subnormal: 2^(1-bias) * 0.m
        return sign * (man_field / 2.0)
    return sign * (2.0 ** (exp_field - 1)) * (1.0 + man_field / 2.0)


E2M1_TABLE = np.array([_e2m1_decode_code(c) for c in range(16)], dtype=np.float64)
MX_BLOCK = 32


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, any integer dtype) -> float64 values."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(e - 127); 0xFF gives NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 0xFF, np.nan, v)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes, element 2i from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix -> float64: element value times its block's E8M0 scale.
    packed [R][K/2] bytes, scales [R][K/32] bytes."""
    v = e2m1_decode(unpack_fp4(packed))                          # [R][K]
    s = e8m0_decode(scales)                                      # [R][K/32]
    return v * np.repeat(s, MX_BLOCK, axis=-1)
