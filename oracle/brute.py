"""Brute-force check of the layer for tiny inputs: for every token, run EVERY
expert's FFN, then mask by the top-k selection and weight by the renormalised
gate. No grouping, no permutation, no matrix routines: plain Python loops over
scalars, so it shares no structure with `oracle.moe`.

TEST INFRASTRUCTURE (used only by the CPU test suite to pin the oracle).

It uses the FP8 codec from `oracle.codecs`, which is pinned on its own against
the format's definition and against an independent library cast.
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


def _expert_out(xrow, w13, w13_scale, w2, w2_scale, fp8: bool):
    """One expert on one token, scalar by scalar."""
    twoF, d = len(w13), len(w13[0])
    F = twoF // 2
    if fp8:
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
            acc = 0.0
            for b0, vals, s in blocks:
                part = 0.0
                for i, hv in enumerate(vals):
                    part += hv * codecs.E4M3_TABLE[w2[m][b0 + i]]
                acc += s * part
            out.append(acc * float(w2_scale[m]))
    else:
        for m in range(len(w2)):
            out.append(_dot(h, w2[m]))
    return out


def brute_layer(x, w_router, bias, k, experts, shared, fp8: bool):
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
            o = _expert_out(x[t], *experts[e], fp8=fp8)
            m = gate.get(e, 0.0)
            for i in range(len(y)):
                y[i] += m * o[i]
        if shared is not None:
            o = _expert_out(x[t], *shared, fp8=fp8)
            for i in range(len(y)):
                y[i] += o[i]
        ids_all.append(chosen)
        w_all.append([gate[e] for e in chosen])
        y_all.append(y)
    return np.array(ids_all, dtype=np.int32), np.array(w_all), np.array(y_all)
