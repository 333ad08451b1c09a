"""Brute-force check of the layer for tiny inputs: for every token, run EVERY
expert's FFN, then mask by the top-k selection and weight by the renormalised
gate. No grouping, no permutation, no matrix routines: plain Python loops over
scalars, so it shares no structure with `oracle.moe`.

TEST INFRASTRUCTURE (used only by the CPU test suite to pin the oracle).

It uses the FP8 and E2M1 value tables from `oracle.codecs`, which are pinned
on their own against the formats' definitions (OCP spec fixtures) and, for
FP8, against an independent library cast. MXFP4 weights are unpacked here
nibble by nibble and scaled block by block, without the codec's array code.
"""
from __future__ import annotations

import math

import numpy as np

from . import codecs


def _dot(a, b):
    s = 0.0
    for p, q in zip(a, b):
        s += float(p) * float(q)
    return s


def _quant_vec(v):
    """Quantise one vector to E4M3 with one float32 scale (decision in float32)."""
    v32 = [float(np.float32(t)) for t in v]
    amax = max(abs(t) for t in v32) if v32 else 0.0
    s = float(np.float32(np.float32(amax) / np.float32(448.0))) if amax != 0 else 1.0
    codes = [int(codecs.e4m3_encode(np.float32(np.float32(t) / np.float32(s)))) for t in v32]
    vals = [float(codecs.E4M3_TABLE[c]) for c in codes]
    return vals, s


def _mx_row(packed_row, scale_row):
    """One MXFP4 weight row: element i is the E2M1 value of nibble i (low
    nibble first) times 2^(scale of block i // 32 - 127)."""
    vals = []
    for i in range(2 * len(packed_row)):
        byte = int(packed_row[i // 2])
        nib = (byte >> 4) if i % 2 else (byte & 0xF)
        vals.append(float(codecs.E2M1_TABLE[nib]) * 2.0 ** (int(scale_row[i // 32]) - 127))
    return vals


def _expert_out(xrow, w13, w13_scale, w2, w2_scale, fp8: bool, mx: bool = False):
    """One expert on one token, scalar by scalar. fp8: quantised activations
    and E4M3 weights with channel scales; mx: quantised activations and MXFP4
    weights (block scales, no channel scale)."""
    twoF = len(w13)
    F = twoF // 2
    if mx:
        xv, sx = _quant_vec(xrow)
        gu = [_dot(xv, _mx_row(w13[n], w13_scale[n])) * sx for n in range(twoF)]
        fp8 = True
    elif fp8:
        xv, sx = _quant_vec(xrow)
        gu = [_dot(xv, [codecs.E4M3_TABLE[c] for c in w13[n]]) * sx * float(w13_scale[n])
              for n in range(twoF)]
    else:
        gu = [_dot(xrow, w13[n]) for n in range(twoF)]
    h = []
    for n in range(F):
        g, u = gu[n], gu[F + n]
        h.append(g / (1.0 + math.exp(-g)) * u)
    out = []
    if fp8:
        blocks = []
        for b0 in range(0, F, 128):
            vals, s = _quant_vec(h[b0:b0 + 128])
            blocks.append((b0, vals, s))
        for m in range(len(w2)):
            wrow = (_mx_row(w2[m], w2_scale[m]) if mx
                    else [codecs.E4M3_TABLE[c] for c in w2[m]])
            acc = 0.0
            for b0, vals, s in blocks:
                part = 0.0
                for i, hv in enumerate(vals):
                    part += hv * wrow[b0 + i]
                acc += s * part
            out.append(acc if mx else acc * float(w2_scale[m]))
    else:
        for m in range(len(w2)):
            out.append(_dot(h, w2[m]))
    return out


def brute_layer(x, w_router, bias, k, experts, shared, fp8: bool, mxfp4: bool = False):
    """x: [T][d] float64 values; w_router: [E][d] float64 values; experts: list
    of (w13, w13_scale, w2, w2_scale) per routed expert (codes or floats);
    shared: the same tuple or None. Returns (ids [T][k], w [T][k], y [T][d]) with
    y in float64 (not rounded)."""
    T = len(x)
    E = len(w_router)
    ids_all, w_all, y_all = [], [], []
    for t in range(T):
        logits = [_dot(x[t], w_router[e]) + (float(bias[e]) if bias is not None else 0.0)
                  for e in range(E)]
        mx = max(logits)
        ex = [math.exp(l - mx) for l in logits]
        z = sum(ex)
        p = [v / z for v in ex]
        # k rounds of "largest remaining logit, lowest index on ties"
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logits[e] > logits[best]:
                    best = e
            chosen.append(best)
        psum = sum(p[e] for e in chosen)
        gate = {e: p[e] / psum for e in chosen}
        y = [0.0] * len(x[t])
        for e in range(E):  # every expert runs; the mask zeroes the unchosen ones
            o = _expert_out(x[t], *experts[e], fp8=fp8, mx=mxfp4)
            m = gate.get(e, 0.0)
            for i in range(len(y)):
                y[i] += m * o[i]
        if shared is not None:
            o = _expert_out(x[t], *shared, fp8=fp8, mx=mxfp4)
            for i in range(len(y)):
                y[i] += o[i]
        ids_all.append(chosen)
        w_all.append([gate[e] for e in chosen])
        y_all.append(y)
    return np.array(ids_all, dtype=np.int32), np.array(w_all), np.array(y_all)
