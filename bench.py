#!/usr/bin/env python3
"""Throughput of one mixture-of-experts layer forward on one MI355X.

A step is one moe_layer_forward call (router, permutation, grouped gate/up and
down GEMMs over the routed experts plus the shared expert, combine) over one
batch of synthetic tokens already resident in HBM. The default workload is
the 30B-shaped decode step (T=64, d=4096, E=128, top-6, F=1024, one shared
expert, FP8 E4M3 weights, bf16 activations); the 3584-token prefill is timed
as a second, reported workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, published
METRIC = "MoE-layer tokens/s at T=64 decode & T=3584 prefill; % of HBM / FP8 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """HIP events through the runtime that torch already loaded."""

    def __init__(self):
        self.L = C.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]
        self.L.hipGetLastError.restype = C.c_int

    def event(self) -> int:
        e = C.c_void_p()
        if self.L.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def ms(self, a: int, b: int, missing_ok: bool = False):
        self.L.hipEventSynchronize(C.c_void_p(b))
        t = C.c_float()
        if self.L.hipEventElapsedTime(C.byref(t), C.c_void_p(a), C.c_void_p(b)) != 0:
            self.L.hipGetLastError()  # clear the runtime's error state
            if missing_ok:
                return None
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def destroy(self, e: int):
        self.L.hipEventDestroy(C.c_void_p(e))


def accounting(cfg, counts):
    """Algorithmic bytes and FLOPs of the layer and of the gate/up GEMM launch,
    given the rows per routed expert (`counts`, from the run's own routing)."""
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared
    touched = int((counts > 0).sum())
    groups = touched + (1 if Fs else 0)
    rows = T * k + (T if Fs else 0)

    def wb(r, c):
        """bytes of an [r][c] weight matrix with its scales: E4M3 codes and a
        float32 per row, or MXFP4 (half a byte per element, one E8M0 byte
        per 32 elements)"""
        return r * c // 2 + r * c // 32 if cfg.precision == "mxfp4" else r * c + 4 * r
    # gate/up launch: each touched group's W13 codes + scales once; per row the
    # x codes + scale in and the h codes + block scales out
    up_bytes = touched * wb(2 * F, d) + (wb(2 * Fs, d) if Fs else 0) \
        + rows * (d + 4) + T * k * (F + F // 32) + (T * (Fs + Fs // 32) if Fs else 0)
    up_flops = 2.0 * d * (T * k * 2 * F + (T * 2 * Fs if Fs else 0))
    # whole layer: every touched expert's weights and scales once, router
    # weight, x in, y out; GEMM FLOPs 6 d F per (token, expert) pair
    layer_bytes = touched * (wb(2 * F, d) + wb(d, F)) \
        + ((wb(2 * Fs, d) + wb(d, Fs)) if Fs else 0) + E * d * 2 + 2 * T * d * 2
    layer_flops = 6.0 * d * (T * k * F + (T * Fs if Fs else 0))
    # down launch: each touched group's W2 codes + scales once; per row the h
    # codes + block scales in and the bf16 output row out
    down_bytes = touched * wb(d, F) + (wb(d, Fs) if Fs else 0) \
        + T * k * (F + F // 32 + 2 * d) + (T * (Fs + Fs // 32 + 2 * d) if Fs else 0)
    down_flops = 2.0 * d * (T * k * F + (T * Fs if Fs else 0))
    return dict(touched=touched, groups=groups, rows=rows, up_bytes=up_bytes, up_flops=up_flops,
                down_bytes=down_bytes, down_flops=down_flops,
                layer_bytes=layer_bytes, layer_flops=layer_flops)


def kernel_roofline(name, alg_bytes, flops, us):
    """HBM and FP8 matrix-core fractions of one launch from its algorithmic
    bytes and FLOPs and its average duration (us)."""
    gbs = alg_bytes / (us / 1e6) / 1e9
    tfl = flops / (us / 1e6) / 1e12
    hbm, mfma = gbs / HBM_PEAK_GBS, tfl / FP8_PEAK_TFLOPS
    return {"kernel": name, "bound": "hbm" if hbm >= mfma else "mfma", "avg_launch_us": round(us, 2),
            "alg_bytes_per_launch": int(alg_bytes), "achieved_GBs": round(gbs, 1),
            "hbm_frac": round(hbm, 4), "fp8_flops_per_launch": flops,
            "achieved_TFLOPs": round(tfl, 1), "fp8_mfma_frac": round(mfma, 4)}


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("ffn.hip", "common.h", "pipeline.h"):
        h.update(open(os.path.join(ROOT, "mixture_experts_softmax_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate/up launch from committed counter runs, or None when
    missing or taken on another version of the kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


EVENT_EVERY = 5  # timed steps per gate/up event pair


def time_layer(cfg, steps, warmup, hip):
    import torch

    import mixture_experts_softmax_amd as M
    from mixture_experts_softmax_amd import _lib
    from synthetic import make_layer

    t = time.time()
    lt = make_layer(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: inputs generated in {time.time() - t:.1f}s")
    L = M.MoELayer(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, F_shared=cfg.F_shared,
                   precision=cfg.precision, w_router=lt.w_router, router_bias=lt.router_bias,
                   w13=lt.w13, w13_scale=lt.w13_scale, w2=lt.w2, w2_scale=lt.w2_scale, ws13=lt.ws13,
                   ws13_scale=lt.ws13_scale, ws2=lt.ws2, ws2_scale=lt.ws2_scale)
    T = cfg.T
    s = L.shape(T)
    ws = L.workspace(T, "cuda")
    W = _lib.make_weights(s, **L.tensors)
    x = lt.x
    y = torch.empty_like(x)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    nsteps = len(_lib.MOE_STEPS)
    UP = _lib.MOE_STEPS.index("gate_up")

    for _ in range(warmup):
        _lib.moe_layer_forward(s, W, x, y, ids, gw, ws)
    torch.cuda.synchronize()

    # the gate/up launch of every EVENT_EVERY-th timed step is bracketed by
    # events on the library's stream (an event pair on every step costs ~5.5 us
    # of GPU time per step, 2% of a decode step; every fifth, ~0.3 us)
    timed = list(range(0, steps, EVENT_EVERY))
    ev_a = [hip.event() for _ in timed]
    ev_b = [hip.event() for _ in timed]
    none = [None] * nsteps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % EVENT_EVERY == 0:
            st, sp = list(none), list(none)
            st[UP], sp[UP] = ev_a[i // EVENT_EVERY], ev_b[i // EVENT_EVERY]
            _lib.moe_layer_forward_events(s, W, x, y, ids, gw, ws, st, sp)
        else:
            _lib.moe_layer_forward(s, W, x, y, ids, gw, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    up_ms = sum(hip.ms(a, b) for a, b in zip(ev_a, ev_b)) / len(timed)
    for e in ev_a + ev_b:
        hip.destroy(e)

    # per-step breakdown (separate short loop, every step of the layer path
    # bracketed; its tile lists come from the permutation scan, so it has no
    # separate "tiles" step)
    reps = min(steps, 10)
    steps_here = [j for j, n in enumerate(_lib.MOE_STEPS) if n != "tiles"]
    starts = [[hip.event() if j in steps_here else None for j in range(nsteps)] for _ in range(reps)]
    stops = [[hip.event() if j in steps_here else None for j in range(nsteps)] for _ in range(reps)]
    for i in range(reps):
        _lib.moe_layer_forward_events(s, W, x, y, ids, gw, ws, starts[i], stops[i])
    torch.cuda.synchronize()
    breakdown = {}
    for j in steps_here:
        t = [hip.ms(starts[i][j], stops[i][j]) for i in range(reps)]
        breakdown[_lib.MOE_STEPS[j]] = round(1e3 * sum(t) / reps, 2)
    for row in starts + stops:
        for e in row:
            if e is not None:
                hip.destroy(e)

    # per-call distribution: one event pair around each whole call
    reps = max(20, min(steps, 50))
    ca = [hip.event() for _ in range(reps)]
    cb = [hip.event() for _ in range(reps)]
    for i in range(reps):
        st, sp = list(none), list(none)
        st[0], sp[nsteps - 1] = ca[i], cb[i]
        _lib.moe_layer_forward_events(s, W, x, y, ids, gw, ws, st, sp)
    torch.cuda.synchronize()
    import numpy as np
    per_call = np.array([hip.ms(a, b) * 1e3 for a, b in zip(ca, cb)])
    for e in ca + cb:
        hip.destroy(e)
    pct = {"p10": round(float(np.percentile(per_call, 10)), 2),
           "p50": round(float(np.percentile(per_call, 50)), 2),
           "p90": round(float(np.percentile(per_call, 90)), 2), "calls": reps}

    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=cfg.E)
    acc = accounting(cfg, counts)
    del L, ws, W, x, y
    return dict(ms_step=ms_step, up_ms=up_ms, breakdown_us=breakdown, acc=acc, counts=counts, lt=lt,
                call_us=pct)


def time_overlap(cfg, steps, warmup, hip):
    """Back-to-back layer calls, one stream against moe_layer_forward_overlap
    (the shared expert on a second stream, forked after the router's logits):
    ms per call of each, from events on the main stream around `steps` calls."""
    import torch

    import mixture_experts_softmax_amd as M
    from mixture_experts_softmax_amd import _lib
    from synthetic import make_layer

    lt = make_layer(cfg, device="cuda")
    L = M.MoELayer(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, F_shared=cfg.F_shared,
                   precision=cfg.precision, w_router=lt.w_router, router_bias=lt.router_bias,
                   w13=lt.w13, w13_scale=lt.w13_scale, w2=lt.w2, w2_scale=lt.w2_scale, ws13=lt.ws13,
                   ws13_scale=lt.ws13_scale, ws2=lt.ws2, ws2_scale=lt.ws2_scale)
    T = cfg.T
    s = L.shape(T)
    ws = L.workspace(T, "cuda")
    W = _lib.make_weights(s, **L.tensors)
    x, y = lt.x, torch.empty_like(lt.x)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    hip.L.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
    hip.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
    evs = []
    for _ in range(2):
        e = C.c_void_p()
        hip.L.hipEventCreateWithFlags(C.byref(e), 2)  # no timing
        evs.append(e.value)
    stream = torch.cuda.current_stream().cuda_stream
    calls = {"single": lambda: _lib.moe_layer_forward(s, W, x, y, ids, gw, ws),
             "overlap": lambda: _lib.moe_layer_forward_overlap(s, W, x, y, ids, gw, ws, side,
                                                               evs[0], evs[1])}
    out = {}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        hip.L.hipEventRecord(C.c_void_p(a), C.c_void_p(stream))
        for _ in range(steps):
            fn()
        hip.L.hipEventRecord(C.c_void_p(b), C.c_void_p(stream))
        out[name + "_ms_per_call"] = round(hip.ms(a, b) / steps, 4)
        hip.destroy(a)
        hip.destroy(b)
    for e in evs:
        hip.destroy(e)
    out["speedup"] = round(out["single_ms_per_call"] / out["overlap_ms_per_call"], 3)
    del L, ws, W, x, y, lt
    torch.cuda.empty_cache()
    return out


def time_graph(cfg, steps, warmup, hip):
    """moe_layer_forward captured once into a HIP graph (torch.cuda.CUDAGraph
    on the capturing stream) and replayed: per-replay GPU time from events on
    the replay stream, back-to-back ms per call, and the host time to issue
    one call, eager and replayed."""
    import numpy as np
    import torch

    import mixture_experts_softmax_amd as M
    from mixture_experts_softmax_amd import _lib
    from synthetic import make_layer

    lt = make_layer(cfg, device="cuda")
    L = M.MoELayer(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, F_shared=cfg.F_shared,
                   precision=cfg.precision, w_router=lt.w_router, router_bias=lt.router_bias,
                   w13=lt.w13, w13_scale=lt.w13_scale, w2=lt.w2, w2_scale=lt.w2_scale, ws13=lt.ws13,
                   ws13_scale=lt.ws13_scale, ws2=lt.ws2, ws2_scale=lt.ws2_scale)
    T = cfg.T
    s = L.shape(T)
    ws = L.workspace(T, "cuda")
    W = _lib.make_weights(s, **L.tensors)
    x = lt.x
    y = torch.empty_like(x)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for _ in range(3):
            _lib.moe_layer_forward(s, W, x, y, ids, gw, ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        _lib.moe_layer_forward(s, W, x, y, ids, gw, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    hip.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def per_call(issue, reps):
        ca = [hip.event() for _ in range(reps)]
        cb = [hip.event() for _ in range(reps)]
        for i in range(reps):
            hip.L.hipEventRecord(C.c_void_p(ca[i]), C.c_void_p(stream))
            issue()
            hip.L.hipEventRecord(C.c_void_p(cb[i]), C.c_void_p(stream))
        torch.cuda.synchronize()
        us = np.array([hip.ms(a, b) * 1e3 for a, b in zip(ca, cb)])
        for e in ca + cb:
            hip.destroy(e)
        return {"p10": round(float(np.percentile(us, 10)), 2),
                "p50": round(float(np.percentile(us, 50)), 2),
                "p90": round(float(np.percentile(us, 90)), 2), "calls": reps}

    def back_to_back(issue, reps):
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        hip.L.hipEventRecord(C.c_void_p(a), C.c_void_p(stream))
        h0 = time.perf_counter()
        for _ in range(reps):
            issue()
        h1 = time.perf_counter()
        hip.L.hipEventRecord(C.c_void_p(b), C.c_void_p(stream))
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / reps
        hip.destroy(a)
        hip.destroy(b)
        return ms, (h1 - h0) * 1e6 / reps

    def eager():
        _lib.moe_layer_forward(s, W, x, y, ids, gw, ws)

    for _ in range(warmup):
        g.replay()
        eager()
    reps = max(20, min(steps, 50))
    out = {}
    for name, fn in (("eager", eager), ("graph", g.replay)):
        ms, host_us = back_to_back(fn, steps)
        out[name] = {"ms_per_call": round(ms, 4), "host_us_per_call": round(host_us, 2),
                     "call_us": per_call(fn, reps)}
    del g, L, ws, W, x, y, lt
    torch.cuda.empty_cache()
    return out


def time_chunked(cfg, chunk, steps, warmup, hip):
    """The workload's tokens as consecutive calls of `chunk` tokens (one step =
    all chunks, in order); returns ms per step and per-chunk accounting.
    chunk may also be a list of call sizes that sum to the batch."""
    import numpy as np
    import torch

    import mixture_experts_softmax_amd as M
    from mixture_experts_softmax_amd import _lib
    from synthetic import make_layer

    lt = make_layer(cfg, device="cuda")
    L = M.MoELayer(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, F_shared=cfg.F_shared,
                   precision=cfg.precision, w_router=lt.w_router, router_bias=lt.router_bias,
                   w13=lt.w13, w13_scale=lt.w13_scale, w2=lt.w2, w2_scale=lt.w2_scale, ws13=lt.ws13,
                   ws13_scale=lt.ws13_scale, ws2=lt.ws2, ws2_scale=lt.ws2_scale)
    sizes = list(chunk) if isinstance(chunk, (list, tuple)) else [chunk] * (cfg.T // chunk)
    bounds = np.cumsum([0] + sizes)
    assert bounds[-1] <= cfg.T
    n = len(sizes)
    shapes = [L.shape(c) for c in sizes]
    ws = L.workspace(max(sizes), "cuda")
    W = _lib.make_weights(shapes[0], **L.tensors)
    x = lt.x
    y = torch.empty_like(x)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")

    def step():
        for c in range(n):
            sl = slice(int(bounds[c]), int(bounds[c + 1]))
            _lib.moe_layer_forward(shapes[c], W, x[sl], y[sl], ids[sl], gw[sl], ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = hip.event(), hip.event()
    hip.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    hip.L.hipEventRecord(C.c_void_p(a), C.c_void_p(stream))
    for _ in range(steps):
        step()
    hip.L.hipEventRecord(C.c_void_p(b), C.c_void_p(stream))
    ms = hip.ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    idn = ids.cpu().numpy()
    bytes_sum = flops_sum = 0.0
    for c in range(n):
        counts = np.bincount(idn[bounds[c]:bounds[c + 1]].reshape(-1), minlength=cfg.E)
        ac = accounting(cfg.with_(T=sizes[c]), counts)
        bytes_sum += ac["layer_bytes"]
        flops_sum += ac["layer_flops"]
    del L, ws, W, x, y, lt
    return dict(ms=ms, chunks=n, bytes=bytes_sum, flops=flops_sum)


def time_qk(cfg, steps, warmup, hip, copies=8):
    """moe_qk_norm_rope in place on `copies` separate QKV buffers in turn (their
    total exceeds the 256 MB Infinity Cache at the prefill size, so every call
    streams from HBM); returns us per call, per-call percentiles and the
    algorithmic bytes (q and k heads read and written once, positions,
    weights)."""
    import numpy as np
    import torch

    from mixture_experts_softmax_amd import _lib
    from synthetic.qk import make_qk

    qt = make_qk(cfg, device="cuda")
    bufs = [qt.qkv.clone() for _ in range(copies)]
    s = _lib.qk_shape(cfg.T, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.row, cfg.q_offset, cfg.k_offset,
                      cfg.eps, cfg.theta, cfg.style, qt.qkv.dtype)
    L = _lib.lib()
    args = [(C.byref(s), C.c_void_p(b.data_ptr()), C.c_void_p(qt.positions.data_ptr()),
             C.c_void_p(qt.q_weight.data_ptr()), C.c_void_p(qt.k_weight.data_ptr())) for b in bufs]
    stream = torch.cuda.current_stream().cuda_stream
    sp = C.c_void_p(stream)
    for i in range(warmup):
        _lib._check(L.moe_qk_norm_rope(*args[i % copies], sp), "moe_qk_norm_rope")
    torch.cuda.synchronize()
    hip.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
    ev = [hip.event() for _ in range(steps + 1)]
    for i in range(steps):
        hip.L.hipEventRecord(C.c_void_p(ev[i]), sp)
        L.moe_qk_norm_rope(*args[i % copies], sp)
    hip.L.hipEventRecord(C.c_void_p(ev[steps]), sp)
    torch.cuda.synchronize()
    us = np.array([hip.ms(ev[i], ev[i + 1]) * 1e3 for i in range(steps)])
    for e in ev:
        hip.destroy(e)
    el = 2 if cfg.precision == "bf16" else 4
    alg = 2 * cfg.T * (cfg.n_q + cfg.n_kv) * cfg.head_dim * el + 4 * cfg.T + 2 * cfg.head_dim * el
    mean_us = float(us.mean())
    del bufs
    # reference: torch's elementwise in-place multiply over contiguous buffers
    # of the query and key heads' size, timed the same way (copies in turn,
    # an event between calls) -- a plain read-modify-write pass over the same
    # bytes, the practical floor for this traffic at this size
    nel = cfg.T * (cfg.n_q + cfg.n_kv) * cfg.head_dim
    refs = [torch.ones(nel, dtype=qt.qkv.dtype, device="cuda") for _ in range(copies)]
    for i in range(warmup):
        refs[i % copies].mul_(1.0)
    torch.cuda.synchronize()
    ev = [hip.event() for _ in range(steps + 1)]
    for i in range(steps):
        hip.L.hipEventRecord(C.c_void_p(ev[i]), sp)
        refs[i % copies].mul_(1.0)
    hip.L.hipEventRecord(C.c_void_p(ev[steps]), sp)
    torch.cuda.synchronize()
    ref_us = float(np.mean([hip.ms(ev[i], ev[i + 1]) * 1e3 for i in range(steps)]))
    for e in ev:
        hip.destroy(e)
    del refs, qt
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: T={cfg.T} heads {cfg.n_q}+{cfg.n_kv} x {cfg.head_dim} "
                        f"{cfg.precision} {cfg.style}, in place",
            "us_per_call": round(mean_us, 2),
            "call_us": {"p10": round(float(np.percentile(us, 10)), 2),
                        "p50": round(float(np.percentile(us, 50)), 2),
                        "p90": round(float(np.percentile(us, 90)), 2), "calls": steps},
            "alg_bytes": alg, "GBs": round(alg / (mean_us / 1e6) / 1e9, 1),
            "hbm_frac": round(alg / (mean_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(cfg.T / (mean_us / 1e6), 1),
            "inplace_reference_us": round(ref_us, 2)}


def hbm_copy_probe():
    """Device-to-device copy of 1 GiB (torch's copy kernel), read + write bytes
    per second: a streaming figure measured on this GPU beside the kernels'."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * n / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def summarize(cfg, r):
    a = r["acc"]
    t = r["ms_step"] / 1e3
    # the layer's two GEMM launches against both peaks: gate/up timed by events
    # inside the timed loop, down by the per-step breakdown loop
    roof = {"gate_up": kernel_roofline("gate_up", a["up_bytes"], a["up_flops"], r["up_ms"] * 1e3)}
    if r["breakdown_us"].get("down"):
        roof["down"] = kernel_roofline("down", a["down_bytes"], a["down_flops"], r["breakdown_us"]["down"])
    return {"workload": f"{cfg.name}: T={cfg.T} k={cfg.k} F={cfg.F}", "value": round(cfg.T / t, 1),
            "roofline": roof,
            "unit": "tokens/s", "ms_per_step": round(r["ms_step"], 4),
            "hbm_frac": round(a["layer_bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
            "fp8_mfma_frac": round(a["layer_flops"] / t / 1e12 / FP8_PEAK_TFLOPS, 4),
            "touched_experts": a["touched"], "call_us": r["call_us"],
            "gate_up_us": round(r["up_ms"] * 1e3, 2),
            "gate_up_GBs": round(a["up_bytes"] / (r["up_ms"] / 1e3) / 1e9, 1),
            "gate_up_TFLOPs": round(a["up_flops"] / (r["up_ms"] / 1e3) / 1e12, 1),
            "step_breakdown_us": r["breakdown_us"]}


def cpu_baseline(cfg, lt, n_tokens):
    """The oracle, untouched, on the first n_tokens tokens of the same inputs
    the GPU just ran (host copies of the touched experts made beforehand)."""
    import numpy as np

    from oracle import inputs as oinputs
    from oracle import moe as omoe

    inp = oinputs.layer_inputs(lt, cache_all=True)
    tok = np.arange(n_tokens)
    # host copies of the touched experts are made before the clock starts
    x64 = omoe.activations(inp)[:n_tokens]
    ids = omoe.topk_ids(omoe.router_logits(x64, omoe.router_weight(inp), inp.router_bias), cfg.k)
    for e in np.unique(ids):
        inp.expert(int(e))
    runs = []
    for _ in range(3):  # the median of three runs
        t = time.perf_counter()
        omoe.layer_forward_tokens(inp, tok)
        runs.append(time.perf_counter() - t)
    dt = sorted(runs)[1]
    try:
        import threadpoolctl
        cores = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    return dict(value=round(n_tokens / dt, 3), unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"first {n_tokens} tokens of the {cfg.name} workload (T={cfg.T}), "
                       f"{len(np.unique(ids))} touched experts, {dt:.1f}s of float64 numpy per "
                       f"run, median of 3 runs ({sum(runs):.1f}s in all)")


def cpu_single_core(cfg, lt, n_tokens, reps):
    """The oracle on one host thread (BLAS limited to one thread): median of
    `reps` runs of the first n_tokens tokens of the workload."""
    import numpy as np
    import threadpoolctl

    from oracle import inputs as oinputs
    from oracle import moe as omoe

    inp = oinputs.layer_inputs(lt, cache_all=True)
    tok = np.arange(n_tokens)
    x64 = omoe.activations(inp)[:n_tokens]
    ids = omoe.topk_ids(omoe.router_logits(x64, omoe.router_weight(inp), inp.router_bias), cfg.k)
    for e in np.unique(ids):
        inp.expert(int(e))
    runs = []
    with threadpoolctl.threadpool_limits(1):
        for _ in range(reps):
            t = time.perf_counter()
            omoe.layer_forward_tokens(inp, tok)
            runs.append(time.perf_counter() - t)
    dt = sorted(runs)[len(runs) // 2]
    return dict(value=round(n_tokens / dt, 3), unit="tokens/s", cores=1, kind="oracle",
                us_per_layer=round(dt * 1e6, 1) if n_tokens == cfg.T else None,
                sample=f"first {n_tokens} of the {cfg.T} tokens of the {cfg.name} workload, "
                       f"{len(np.unique(ids))} touched experts, one thread, median of {reps} runs "
                       f"({sum(runs):.1f}s in all)")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "b100", "skew", "decode_mxfp4", "prefill_mxfp4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads (prefill, 100B-shaped, skewed, chunked prefill) "
                         "and the copy probe")
    ap.add_argument("--qk-only", choices=["qk_prefill", "qk_decode"],
                    help="only time the QK-Norm + RoPE step on that workload and print its line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device-to-device copy (counter calibration) and exit")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the workload the CPU oracle runs (0: the whole batch, capped at 64)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by expert across GPUs, which is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        # a plain copy of known size: HBM counters read on its dispatches give
        # the scale between counter units and bytes moved
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    import numpy as np

    from synthetic import CONFIGS
    hip = Hip()
    if args.qk_only:
        from synthetic.qk import QK_CONFIGS
        print(json.dumps({"qk_norm_rope": time_qk(QK_CONFIGS[args.qk_only], args.steps,
                                                  args.warmup, hip)}), flush=True)
        return
    cfg = CONFIGS[args.workload]
    r = time_layer(cfg, args.steps, args.warmup, hip)
    lt = r.pop("lt")
    acc = r["acc"]
    value = cfg.T / (r["ms_step"] / 1e3)
    achieved = acc["up_bytes"] / (r["up_ms"] / 1e3) / 1e9
    traffic = measured_traffic(args.workload)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if cfg.precision == "fp8" else "fp8_e4m3 x mxfp4",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} "
                               f"F={cfg.F} shared F={cfg.F_shared}, "
                               f"{'MXFP4' if cfg.precision == 'mxfp4' else 'FP8 E4M3'} weights, bf16 x",
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "F_shared": cfg.F_shared, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "gate_up_fp8_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "alg_bytes_per_launch": acc["up_bytes"], "avg_launch_us": round(r["up_ms"] * 1e3, 2)},
        "layer": {"alg_bytes": acc["layer_bytes"], "fp8_flops": acc["layer_flops"],
                  "hbm_frac": round(acc["layer_bytes"] / (r["ms_step"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "fp8_mfma_frac": round(acc["layer_flops"] / (r["ms_step"] / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                  "touched_experts": acc["touched"], "step_breakdown_us": r["breakdown_us"]},
    }
    out["layer"]["call_us"] = r["call_us"]
    out["layer"]["kernels"] = summarize(cfg, r)["roofline"]
    if not args.no_secondary:
        # the other workloads, reported beside the headline (not part of `value`)
        # at least 50 warm-up steps: after the seconds of input generation the
        # first few hundred microseconds of GPU work run slower (prefill: 598 us
        # per timed step after 5 warm-up steps, 546 after 50, 542 per call)
        sec_steps, sec_warm = max(5, args.steps // 2), max(50, args.warmup)
        for name in ("prefill", "b100", "skew", "decode_mxfp4", "prefill_mxfp4"):
            if name == args.workload:
                continue
            c2 = CONFIGS[name]
            log(f"[bench] secondary workload {name}")
            r2 = time_layer(c2, sec_steps, sec_warm, hip)
            del r2["lt"]
            out[name] = summarize(c2, r2)
            if name == "skew":
                nz = r2["counts"][r2["counts"] > 0]
                out[name]["group_rows"] = {"empty": int((r2["counts"] == 0).sum()),
                                           "min": int(nz.min()), "median": int(np.median(nz)),
                                           "max": int(nz.max())}
            torch.cuda.empty_cache()
        p = CONFIGS["prefill"]
        log("[bench] secondary workload prefill in 256-token chunks")
        rc = time_chunked(p, 256, sec_steps, sec_warm, hip)
        t = rc["ms"] / 1e3
        out["prefill_chunked"] = {
            "workload": f"prefill: T={p.T} as {rc['chunks']} calls of 256 tokens",
            "value": round(p.T / t, 1), "unit": "tokens/s", "ms_per_step": round(rc["ms"], 4),
            "us_per_chunk": round(rc["ms"] * 1e3 / rc["chunks"], 2),
            "hbm_frac": round(rc["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
            "fp8_mfma_frac": round(rc["flops"] / t / 1e12 / FP8_PEAK_TFLOPS, 4)}
        torch.cuda.empty_cache()
        # mixed batch: 256 prefill-chunk tokens and 32 decode tokens in one
        # call, against the same tokens as two calls (256, then 32)
        mx_cfg = CONFIGS["mixed"]
        log("[bench] secondary workload mixed (one call vs 256 + 32)")
        rm = time_layer(mx_cfg, sec_steps, sec_warm, hip)
        del rm["lt"]
        out["mixed"] = summarize(mx_cfg, rm)
        torch.cuda.empty_cache()
        rs = time_chunked(mx_cfg, [256, 32], sec_steps, sec_warm, hip)
        out["mixed"]["split_256_32_ms"] = round(rs["ms"], 4)
        out["mixed"]["speedup_vs_split"] = round(rs["ms"] / rm["ms_step"], 3)
        torch.cuda.empty_cache()
        # the shared expert overlapped with the routing on a second stream
        for name in ("decode", "prefill"):
            log(f"[bench] {name}: shared expert on a second stream")
            out.setdefault(name if name != cfg.name else "layer", {})["shared_overlap"] = \
                time_overlap(CONFIGS[name], sec_steps, sec_warm, hip)
        # the decode step captured into a HIP graph and replayed
        log("[bench] decode replayed from a HIP graph")
        out["decode_graph"] = time_graph(cfg if cfg.T <= 64 else CONFIGS["decode"],
                                         sec_steps * 2, sec_warm, hip)
        # the step before the layer's attention: QK-Norm + RoPE in place
        from synthetic.qk import QK_CONFIGS
        for qn in ("qk_prefill", "qk_decode"):
            log(f"[bench] secondary workload {qn}")
            out[qn] = time_qk(QK_CONFIGS[qn], 50, 5, hip)
        out["hbm_copy_probe_GBs"] = hbm_copy_probe()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        n = args.cpu_tokens if args.cpu_tokens > 0 else min(cfg.T, 64)
        out["cpu_baseline"] = cpu_baseline(cfg, lt, n)
        # the same oracle on one host thread: the whole tiny workload, and a
        # sample of the decode step
        from synthetic import make_layer
        log("[bench] timing the CPU oracle on one thread")
        tiny = CONFIGS["tiny"]
        lt_tiny = make_layer(tiny, device="cuda")
        single = {"tiny": cpu_single_core(tiny, lt_tiny, tiny.T, 21)}
        if cfg.name == "decode":
            single["decode"] = cpu_single_core(cfg, lt, 8, 3)
        out["cpu_baseline"]["single_core"] = single
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
