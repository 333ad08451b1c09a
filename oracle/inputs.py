"""Glue between the synthetic input tensors and the oracle.

TEST INFRASTRUCTURE (tests, smoke check, benchmark CPU baseline only).

`layer_inputs` copies a generated layer to host numpy arrays in their stored
formats; expert weights are copied one expert at a time, on demand, so a
full-size layer that lives on the GPU is never copied whole. `HOOKS` gives the
input generator the oracle's routing decisions for near-tie redraws and skew
calibration.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe


def _np(t):
    if t is None:
        return None
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy().copy()
    return t.numpy().copy()


def layer_inputs(lt, cache_all: bool = False) -> moe.LayerInputs:
    """cache_all keeps every expert copied so far (else at most 8 are held)."""
    cfg = lt.cfg
    quant = cfg.precision != "f32"
    fmt = "mxfp4" if cfg.precision == "mxfp4" else "fp8"
    cache = {}

    def expert(e: int) -> moe.ExpertWeights:
        if e not in cache:
            if len(cache) > 8 and not cache_all:
                cache.clear()
            cache[e] = moe.ExpertWeights(
                _np(lt.w13[e]), _np(lt.w13_scale[e]) if quant else None,
                _np(lt.w2[e]), _np(lt.w2_scale[e]) if quant else None, fmt)
        return cache[e]

    shared = None
    if lt.ws13 is not None:
        shared = moe.ExpertWeights(_np(lt.ws13), _np(lt.ws13_scale) if quant else None,
                                   _np(lt.ws2), _np(lt.ws2_scale) if quant else None, fmt)
    return moe.LayerInputs(
        precision=cfg.precision, x=_np(lt.x), w_router=_np(lt.w_router),
        router_bias=_np(lt.router_bias), k=cfg.k, E=cfg.E, expert=expert, shared=shared)


class _Hooks:
    """Routing decisions for the input generator, made by the oracle."""

    @staticmethod
    def near_tie(x, w_router, bias, k, min_gap):
        return moe.near_tie_rows(moe.router_logits(x, w_router, bias), k, min_gap)

    @staticmethod
    def expert_counts(x, w_router, bias, k, E):
        ids = moe.topk_ids(moe.router_logits(x, w_router, bias), k)
        return np.bincount(ids.reshape(-1), minlength=E)


HOOKS = _Hooks()
