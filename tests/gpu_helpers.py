"""Shared pieces of the GPU tests: build a layer from generated tensors, run
the library through its C ABI, copy results back, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_softmax_amd as moe_lib
from mixture_experts_softmax_amd import _lib
from oracle import codecs
from oracle import inputs as oinputs
from oracle import moe as omoe
from synthetic import LayerTensors, make_layer

DEV = "cuda"

# Tolerances against the float64 oracle.
FP8_MAX_ABS, FP8_REL_L2 = 2e-2, 1e-2
F32_MAX_ABS, F32_REL_L2 = 1e-5, 1e-5
W_MAX_ABS = 1e-5


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gen(cfg, **kw) -> LayerTensors:
    return make_layer(cfg, device=DEV, hooks=oinputs.HOOKS, **kw)


def layer(lt: LayerTensors) -> moe_lib.MoELayer:
    c = lt.cfg
    return moe_lib.MoELayer(d=c.d, E=c.E, k=c.k, F=c.F, F_shared=c.F_shared, precision=c.precision,
                            w_router=lt.w_router, router_bias=lt.router_bias, w13=lt.w13,
                            w13_scale=lt.w13_scale, w2=lt.w2, w2_scale=lt.w2_scale, ws13=lt.ws13,
                            ws13_scale=lt.ws13_scale, ws2=lt.ws2, ws2_scale=lt.ws2_scale)


def run_layer(lt: LayerTensors, x=None):
    """Whole layer through moe_layer_forward; returns host (ids, w, y as float64)."""
    c = lt.cfg
    x = lt.x if x is None else x
    T = x.shape[0]
    ids = torch.full((T, c.k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, c.k), -1.0, dtype=torch.float32, device=DEV)
    y = layer(lt).forward(x, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), y.to(torch.float64).cpu().numpy()


def shape_of(c, T=None):
    return _lib.shape(c.T if T is None else T, c.d, c.E, c.k, c.F, c.F_shared, c.precision)


def compare_y(y_gpu: np.ndarray, y_ref: np.ndarray, precision: str, what: str = "y"):
    diff = np.abs(y_gpu - y_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    den = float(np.sqrt((y_ref ** 2).sum()))
    rel = float(np.sqrt((diff ** 2).sum()) / den) if den > 0 else max_abs
    lim_abs, lim_rel = (FP8_MAX_ABS, FP8_REL_L2) if precision == "fp8" else (F32_MAX_ABS, F32_REL_L2)
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (limits {lim_abs:g}, {lim_rel:g})")
    assert max_abs <= lim_abs, f"{what}: max abs err {max_abs} > {lim_abs}"
    assert rel <= lim_rel, f"{what}: rel-L2 err {rel} > {lim_rel}"
    return max_abs, rel


def check_routing_invariants(ids: np.ndarray, w: np.ndarray, E: int):
    T, k = ids.shape
    assert np.all((ids >= 0) & (ids < E))
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    assert np.allclose(w.sum(1), 1.0, atol=1e-5)
    assert np.all(np.diff(w, axis=1) <= 1e-6)  # descending gate order
