"""Pins for the oracle's number formats (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_spec.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_spec_values():
    for code, val in _golden():
        got = codecs.E4M3_TABLE[code]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_table_structure():
    t = codecs.E4M3_TABLE
    finite = ~np.isnan(t)
    assert finite.sum() == 254                    # only S.1111.111 is NaN
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)               # codes order the values
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])  # sign-magnitude
    # subnormals are k * 2^-9, normals step by 2^(e-3) in each binade
    assert np.array_equal(pos[:8], np.arange(8) * 2.0 ** -9)
    for e in range(1, 16):
        binade = pos[8 * e: 8 * e + 8]
        expect = 2.0 ** (e - 7) * (1 + np.arange(len(binade)) / 8.0)
        assert np.array_equal(binade, expect)


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in codecs.E4M3_NAN_CODES], dtype=np.uint8)
    assert np.array_equal(codecs.e4m3_encode(codecs.e4m3_decode(codes)), codes)


def test_e4m3_midpoints_round_to_even():
    pos = codecs.E4M3_TABLE[:0x7F]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2
        want = c if c % 2 == 0 else c + 1
        assert codecs.e4m3_encode(np.array([mid]))[0] == want
        assert codecs.e4m3_encode(np.array([-mid]))[0] == (want | 0x80)
        eps = (hi - lo) * 1e-6
        assert codecs.e4m3_encode(np.array([mid - eps]))[0] == c
        assert codecs.e4m3_encode(np.array([mid + eps]))[0] == c + 1


def test_e4m3_saturation_and_signed_zero():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e30, -500.0, -1e-9, 1e-9, 0.0, -0.0])
    got = codecs.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x80]
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.inf]))


def test_e4m3_matches_torch_cast():
    """Independent library routine: torch's float8_e4m3fn cast (RNE) on float32
    values inside the finite range, plus every midpoint and its neighbours."""
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.standard_normal(200_000) * 0.05,
        rng.standard_normal(50_000) * 1e-3,
    ]).astype(np.float32)
    pos = codecs.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    ours = codecs.e4m3_encode(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(300_000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    # values exactly halfway between two bf16 numbers
    base = torch.from_numpy(rng.standard_normal(10_000).astype(np.float32)).to(torch.bfloat16)
    b32 = base.to(torch.float32).numpy().view(np.uint32)
    halves = (b32 + np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, halves, -halves])
    ours = codecs.bf16_encode(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, theirs)
    assert np.array_equal(codecs.bf16_decode(theirs), torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy())


def test_bf16_round_direct_from_float64():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even -> 1.0;
    # a hair above must go up (float32 double rounding would lose the hair).
    assert codecs.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert codecs.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert codecs.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


MX_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_e8m0_ocp_mx_spec.txt")


def test_mx_spec_values():
    """Every E2M1 code and the E8M0 boundary codes equal the OCP MX spec's."""
    n = 0
    for line in open(MX_GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        fmt, code, val = line.split()
        got = codecs.E2M1_TABLE[int(code, 16)] if fmt == "E2M1" else codecs.e8m0_decode(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (fmt, code, got)
        n += 1
    assert n == 21


def test_e2m1_structure():
    """Magnitudes increase with the code, the sign bit mirrors them, and the
    spacing doubles from one binade to the next (one mantissa bit)."""
    pos = codecs.E2M1_TABLE[:8]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(codecs.E2M1_TABLE[8:], -pos)
    assert np.array_equal(np.diff(pos), [0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0])


def test_unpack_fp4_low_nibble_first():
    p = np.array([[0x21, 0xF0, 0x9A]], np.uint8)
    assert codecs.unpack_fp4(p).tolist() == [[1, 2, 0, 15, 10, 9]]
