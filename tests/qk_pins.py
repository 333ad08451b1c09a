"""Pins of the QK-Norm + RoPE oracle (oracle/qk_rope.py) to things other than
itself: the rotation written as a complex exponential, torch's RMSNorm, a
scalar brute-force loop, closed forms and RoPE's relative-position property.
Each returns None or raises AssertionError; test_oracle_qk.py runs them and
re-runs them against planted mistakes."""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as tF

from oracle import qk_rope


def _rng(seed):
    return np.random.default_rng(seed)


def _complex_rope(x, pos, theta, style):
    """The rotation as multiplication of a + ib by exp(i p f), f computed as
    exp(-(2i/hd) ln theta)."""
    hd = x.shape[-1]
    h = hd // 2
    if style == "interleaved":
        z = x[..., 0::2] + 1j * x[..., 1::2]
    else:
        z = x[..., :h] + 1j * x[..., h:]
    f = np.exp(-(2.0 * np.arange(h) / hd) * math.log(theta))
    z = z * np.exp(1j * np.asarray(pos, np.float64)[:, None, None] * f[None, None, :])
    out = np.empty_like(x)
    if style == "interleaved":
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        out[..., :h], out[..., h:] = z.real, z.imag
    return out


def pin_rope_is_complex_rotation():
    rng = _rng(300)
    for style in qk_rope.STYLES:
        for hd, theta in [(8, 10000.0), (64, 500000.0), (128, 10000.0), (6, 3.0)]:
            x = rng.standard_normal((5, 3, hd))
            pos = rng.integers(0, 40000, 5)
            got = qk_rope.rope(x, pos, theta, style)
            assert np.allclose(got, _complex_rope(x, pos, theta, style), rtol=0, atol=1e-9), (style, hd)


def pin_rope_closed_forms():
    for style in qk_rope.STYLES:
        # one pair, frequency 1: position p turns (1, 0) by p radians
        for p in (0, 1, 2, 7, 1000):
            got = qk_rope.rope(np.array([[[1.0, 0.0]]]), np.array([p]), 10000.0, style)
            assert np.allclose(got[0, 0], [math.cos(p), math.sin(p)], atol=1e-12)
        # second pair of a 4-wide head at theta 100: frequency 100^(-1/2) = 0.1,
        # so position 10 turns it by exactly one radian; the first pair by 10
        x = np.zeros((1, 1, 4))
        ia, ib = qk_rope.pair_views(4, style)
        x[0, 0, ia[1]] = 1.0
        x[0, 0, ia[0]] = 1.0
        got = qk_rope.rope(x, np.array([10]), 100.0, style)[0, 0]
        assert abs(got[ia[1]] - math.cos(1.0)) < 1e-12 and abs(got[ib[1]] - math.sin(1.0)) < 1e-12
        assert abs(got[ia[0]] - math.cos(10.0)) < 1e-12 and abs(got[ib[0]] - math.sin(10.0)) < 1e-12
        # position 0 is the identity
        x = _rng(301).standard_normal((2, 4, 16))
        assert np.array_equal(qk_rope.rope(x, np.zeros(2, np.int64), 10000.0, style), x)


def pin_rope_invariants():
    rng = _rng(302)
    for style in qk_rope.STYLES:
        hd = 32
        x = rng.standard_normal((6, 2, hd))
        pos = rng.integers(-5000, 5000, 6)
        y = qk_rope.rope(x, pos, 10000.0, style)
        ia, ib = qk_rope.pair_views(hd, style)
        # a rotation keeps each pair's length, and turning back undoes it
        assert np.allclose(x[..., ia] ** 2 + x[..., ib] ** 2, y[..., ia] ** 2 + y[..., ib] ** 2, atol=1e-12)
        assert np.allclose(qk_rope.rope(y, -pos, 10000.0, style), x, atol=1e-12)
        # relative position: <R(m) q, R(n) k> depends on m - n only
        q = rng.standard_normal((1, 1, hd))
        k = rng.standard_normal((1, 1, hd))
        for m, n, s in [(5, 2, 11), (100, 900, 37), (0, 3000, 1234)]:
            d1 = np.sum(qk_rope.rope(q, np.array([m]), 10000.0, style) *
                        qk_rope.rope(k, np.array([n]), 10000.0, style))
            d2 = np.sum(qk_rope.rope(q, np.array([m + s]), 10000.0, style) *
                        qk_rope.rope(k, np.array([n + s]), 10000.0, style))
            assert abs(d1 - d2) < 1e-9


def pin_rms_norm():
    rng = _rng(303)
    for hd, eps in [(8, 1e-6), (64, 0.5), (128, 1e-5)]:
        x = rng.standard_normal((4, 3, hd))
        w = 1.0 + 0.3 * rng.standard_normal(hd)
        ref = tF.rms_norm(torch.from_numpy(x), (hd,), weight=torch.from_numpy(w), eps=eps).numpy()
        assert np.allclose(qk_rope.rms_norm_heads(x, w, eps), ref, rtol=1e-12, atol=1e-14)
    # closed forms with eps = 0: a constant vector maps to the weight (times
    # its sign); (3, 4) has rms sqrt(12.5); the norm ignores scale
    w = np.array([0.5, 2.0, -1.0, 3.0])
    assert np.allclose(qk_rope.rms_norm_heads(np.full(4, -2.5), w, 0.0), -w, atol=1e-15)
    assert np.allclose(qk_rope.rms_norm_heads(np.array([3.0, 4.0]), np.ones(2), 0.0),
                       [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], atol=1e-15)
    x = rng.standard_normal(16)
    assert np.allclose(qk_rope.rms_norm_heads(7.25 * x, np.ones(16), 0.0),
                       qk_rope.rms_norm_heads(x, np.ones(16), 0.0), atol=1e-14)
    # a zero head stays zero
    assert np.array_equal(qk_rope.rms_norm_heads(np.zeros(8), np.ones(8), 1e-6), np.zeros(8))


def _brute(qkv, pos, qw, kw, n_q, n_kv, hd, qo, ko, eps, theta, style):
    """Element by element: per head, the mean square, the scaled values, then
    each pair turned by its angle."""
    out = [list(map(float, row)) for row in qkv]
    for t in range(len(out)):
        for off, nh, w in ((qo, n_q, qw), (ko, n_kv, kw)):
            for h in range(nh):
                base = off + h * hd
                vals = [out[t][base + i] for i in range(hd)]
                ms = sum(v * v for v in vals) / hd
                r = math.sqrt(ms + eps)
                nv = [vals[i] / r * float(w[i]) for i in range(hd)]
                for i in range(hd // 2):
                    if style == "interleaved":
                        ia, ib = 2 * i, 2 * i + 1
                    else:
                        ia, ib = i, i + hd // 2
                    ang = float(pos[t]) * float(theta) ** (-2.0 * i / hd)
                    a, b = nv[ia], nv[ib]
                    out[t][base + ia] = a * math.cos(ang) - b * math.sin(ang)
                    out[t][base + ib] = a * math.sin(ang) + b * math.cos(ang)
    return np.array(out)


def pin_qk_vs_brute():
    rng = _rng(304)
    for style in qk_rope.STYLES:
        for T, n_q, n_kv, hd, pad in [(3, 2, 1, 8, 0), (2, 3, 2, 4, 5), (4, 1, 1, 6, 2)]:
            row = (n_q + 2 * n_kv) * hd + pad
            qo, ko = pad, pad + n_q * hd  # some leading columns before q
            qkv = rng.standard_normal((T, row + pad))
            pos = rng.integers(0, 5000, T)
            qw = 1.0 + 0.2 * rng.standard_normal(hd)
            kw = 1.0 + 0.2 * rng.standard_normal(hd)
            args = (pos, qw, kw, n_q, n_kv, hd, qo, ko, 1e-3, 10000.0, style)
            got = qk_rope.qk_norm_rope(qkv, *args)
            ref = _brute(qkv, *args)
            assert np.allclose(got, ref, rtol=0, atol=1e-12), (style, T, n_q, n_kv, hd)
            # columns outside the q and k heads are untouched
            keep = np.ones(qkv.shape[1], bool)
            keep[qo:qo + n_q * hd] = False
            keep[ko:ko + n_kv * hd] = False
            assert np.array_equal(got[:, keep], qkv[:, keep])


def pin_qk_vs_torch():
    """Torch's RMSNorm and a polar-form rotation on a model-sized row."""
    rng = _rng(305)
    T, n_q, n_kv, hd = 3, 32, 4, 128
    qkv = rng.standard_normal((T, (n_q + 2 * n_kv) * hd))
    pos = np.array([0, 3583, 3700])
    qw = 1.0 + 0.2 * rng.standard_normal(hd)
    kw = 1.0 + 0.2 * rng.standard_normal(hd)
    for style in qk_rope.STYLES:
        got = qk_rope.qk_norm_rope(qkv, pos, qw, kw, n_q, n_kv, hd, 0, n_q * hd, 1e-6, 1e6, style)
        x = torch.from_numpy(qkv)
        for off, nh, w in ((0, n_q, qw), (n_q * hd, n_kv, kw)):
            hs = x[:, off:off + nh * hd].reshape(T, nh, hd)
            n = tF.rms_norm(hs, (hd,), weight=torch.from_numpy(w), eps=1e-6)
            f = torch.pow(torch.tensor(1e6, dtype=torch.float64), -torch.arange(0, hd, 2, dtype=torch.float64) / hd)
            rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64),
                              torch.from_numpy(pos).double()[:, None] * f[None, :])[:, None, :]
            if style == "interleaved":
                z = torch.view_as_complex(n.reshape(T, nh, hd // 2, 2).contiguous()) * rot
                r = torch.view_as_real(z).reshape(T, nh, hd)
            else:
                z = torch.complex(n[..., :hd // 2], n[..., hd // 2:]) * rot
                r = torch.cat([z.real, z.imag], dim=-1)
            assert np.allclose(got[:, off:off + nh * hd], r.reshape(T, -1).numpy(), rtol=0, atol=1e-10), style
        assert np.array_equal(got[:, (n_q + n_kv) * hd:], qkv[:, (n_q + n_kv) * hd:])


ALL = [pin_rope_is_complex_rotation, pin_rope_closed_forms, pin_rope_invariants, pin_rms_norm,
       pin_qk_vs_brute, pin_qk_vs_torch]
