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


def run_layer(lt: LayerTensors, x=None, inter: bool = False):
    """Whole layer through moe_layer_forward; returns host (ids, w, y as
    float64), and with inter=True also a dict of the layer's own intermediate
    results read back from its workspace (the keys run_stepwise uses)."""
    c = lt.cfg
    x = lt.x if x is None else x
    T = x.shape[0]
    ids = torch.full((T, c.k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, c.k), -1.0, dtype=torch.float32, device=DEV)
    L = layer(lt)
    y = L.forward(x, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    out = (ids.cpu().numpy(), w.cpu().numpy(), y.to(torch.float64).cpu().numpy())
    if not inter:
        return out
    mid = {n: t.cpu() for n, t in L.intermediates(T).items()}
    st = dict(ids=out[0], w=out[1], y=out[2],
              xq=mid["xq"].numpy() if "xq" in mid else None,
              xs=mid["x_scale"].numpy() if "x_scale" in mid else None,
              offsets=mid["offsets"].numpy(), sorted_pair=mid["sorted_pair"].numpy(),
              pair_to_row=mid["pair_to_row"].numpy(), h=mid["h"].numpy(),
              hs=mid["h_scale"].numpy() if "h_scale" in mid else None,
              h_sh=mid["h_shared"].numpy() if "h_shared" in mid else None,
              hs_sh=mid["h_shared_scale"].numpy() if "h_shared_scale" in mid else None,
              eo=mid["expert_out"].to(torch.float64).numpy())
    return out + (st,)


def check_permutation(st: dict, ids_ref: np.ndarray, E: int, what: str = "layer"):
    """offsets, sorted_pair and pair_to_row bit-exact against the oracle's
    permutation of the oracle's expert ids."""
    P = omoe.permute(ids_ref, E)
    assert np.array_equal(st["offsets"], P.offsets), f"{what}: offsets differ"
    assert np.array_equal(st["sorted_pair"], P.sorted_pair), f"{what}: sorted_pair differs"
    assert np.array_equal(st["pair_to_row"], P.pair_to_row), f"{what}: pair_to_row differs"


def shape_of(c, T=None):
    return _lib.shape(c.T if T is None else T, c.d, c.E, c.k, c.F, c.F_shared, c.precision)


def run_stepwise(lt: LayerTensors, x=None):
    """The layer through the separate entry points (route, permute, grouped FFN
    over the routed experts, grouped FFN over the shared expert, combine),
    keeping every intermediate; returns host numpy arrays."""
    c = lt.cfg
    x = lt.x if x is None else x
    T, d, E, k, F, Fs = x.shape[0], c.d, c.E, c.k, c.F, c.F_shared
    fp8 = c.precision != "f32"
    s = shape_of(c, T)
    i32, f32 = torch.int32, torch.float32
    ids = torch.empty((T, k), dtype=i32, device=DEV)
    w = torch.empty((T, k), dtype=f32, device=DEV)
    xq = torch.empty((T, d), dtype=torch.uint8, device=DEV) if fp8 else None
    xs = torch.empty((T,), dtype=f32, device=DEV) if fp8 else None
    _lib.moe_route_topk(s, x, lt.w_router, lt.router_bias, ids, w, xq, xs,
                        moe_lib.alloc_workspace(_lib.moe_route_workspace_size(s), DEV))
    off = torch.empty(E + 1, dtype=i32, device=DEV)
    sp = torch.empty(T * k, dtype=i32, device=DEV)
    p2r = torch.empty(T * k, dtype=i32, device=DEV)
    _lib.moe_permute(s, ids, off, sp, p2r, moe_lib.alloc_workspace(_lib.moe_permute_workspace_size(s), DEV))
    odt = torch.bfloat16 if fp8 else f32
    hdt = torch.uint8 if fp8 else f32
    a, a_s = (xq, xs) if fp8 else (x, None)

    def ffn(G, offsets, row_src, div, rows, FF, w13, s13, w2, s2):
        out = torch.empty((rows, d), dtype=odt, device=DEV)
        h = torch.empty((rows, FF), dtype=hdt, device=DEV)
        hs = torch.empty((rows, FF // 128), dtype=f32, device=DEV) if fp8 else None
        f = _lib.make_ffn(d, FF, G, rows, c.precision, offsets, row_src, div, a, a_s, w13, s13, w2, s2,
                          out, h, hs)
        _lib.moe_grouped_ffn(f, moe_lib.alloc_workspace(_lib.moe_grouped_ffn_workspace_size(f), DEV))
        return out, h, hs
    eo, h, hs = ffn(E, off, sp, k, T * k, F, lt.w13, lt.w13_scale, lt.w2, lt.w2_scale)
    so = hsh = hssh = None
    if Fs:
        so, hsh, hssh = ffn(1, torch.tensor([0, T], dtype=i32, device=DEV), None, 1, T, Fs,
                            lt.ws13, lt.ws13_scale, lt.ws2, lt.ws2_scale)
    y = torch.empty((T, d), dtype=odt, device=DEV)
    _lib.moe_combine(s, eo, p2r, w, so, y)
    torch.cuda.synchronize()

    return dict(ids=ids.cpu().numpy(), w=w.cpu().numpy(), xq=None if xq is None else xq.cpu().numpy(),
                xs=None if xs is None else xs.cpu().numpy(), offsets=off.cpu().numpy(),
                sorted_pair=sp.cpu().numpy(), pair_to_row=p2r.cpu().numpy(),
                eo=eo.to(torch.float64).cpu().numpy(), h=h.cpu().numpy(),
                hs=None if hs is None else hs.cpu().numpy(),
                so=None if so is None else so.to(torch.float64).cpu().numpy(),
                h_sh=None if hsh is None else hsh.cpu().numpy(),
                hs_sh=None if hssh is None else hssh.cpu().numpy(),
                y=y.to(torch.float64).cpu().numpy())


def compare_y(y_gpu: np.ndarray, y_ref: np.ndarray, precision: str, what: str = "y",
              extra_abs=0.0):
    """y_ref is the oracle's float64 value before any output rounding.
    extra_abs (scalar or elementwise) widens the max-abs bound where validated
    quantisation decisions of the kernel differ from the oracle's."""
    diff = np.abs(y_gpu - y_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    den = float(np.sqrt((y_ref ** 2).sum()))
    rel = float(np.sqrt((diff ** 2).sum()) / den) if den > 0 else max_abs
    lim_abs, lim_rel = (FP8_MAX_ABS, FP8_REL_L2) if precision != "f32" else (F32_MAX_ABS, F32_REL_L2)
    lim = lim_abs + np.asarray(extra_abs, np.float64)
    widened = int((diff > lim_abs).sum())
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (limits {lim_abs:g}, {lim_rel:g}); "
        f"{widened} of {diff.size} outputs beyond {lim_abs:g}, each within its validated-decision bound")
    bad = diff > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs exceed their bound (max abs err {max_abs})"
    assert rel <= lim_rel, f"{what}: rel-L2 err {rel} > {lim_rel}"
    return max_abs, rel


def fp8_bounds(inp, st, tokens=None):
    """Validate the kernel's h decisions (routed groups and shared expert) for
    the given tokens (default: all) against the oracle's exact h; return the
    elementwise extra bound for y [len(tokens)][d], the extra bound for
    expert_out rows {row: [d]} and for shared_out [len(tokens)][d], and the
    number of neighbouring-code decisions."""
    from tests import fp8_checks as FC
    k = inp.k
    T = st["ids"].shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    d = st["y"].shape[1]
    x64 = omoe.activations(inp)[tokens]
    xq, sx = omoe.quantize_rows_e4m3(x64)
    ids = st["ids"][tokens]
    p2r = st["pair_to_row"]
    row_bound = {}
    flips = codes = 0
    for e in np.unique(ids):
        sel = np.argwhere(ids == e)           # (token index, slot)
        ew = inp.expert(int(e))
        rows = p2r[tokens[sel[:, 0]] * k + sel[:, 1]]
        n, dhq = FC.validate_h(xq[sel[:, 0]], sx[sel[:, 0]], ew, st["h"][rows], st["hs"][rows])
        flips += n
        codes += st["h"][rows].size
        eff = FC.down_effect(dhq, ew)
        for i, r in enumerate(rows):
            row_bound[int(r)] = eff[i]
    extra = np.zeros((len(tokens), d))
    w = st["w"][tokens]
    for i, t in enumerate(tokens):
        for j in range(k):
            extra[i] += w[i, j] * row_bound[int(p2r[t * k + j])]
    shared_extra = None
    if inp.shared is not None:
        n, dhq = FC.validate_h(xq, sx, inp.shared, st["h_sh"][tokens], st["hs_sh"][tokens])
        flips += n
        codes += st["h_sh"][tokens].size
        shared_extra = FC.down_effect(dhq, inp.shared)
        extra += shared_extra
    FC.check_flip_rate(flips, codes)
    return extra, row_bound, shared_extra, flips


def check_routing_invariants(ids: np.ndarray, w: np.ndarray, E: int):
    T, k = ids.shape
    assert np.all((ids >= 0) & (ids < E))
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    assert np.allclose(w.sum(1), 1.0, atol=1e-5)
    assert np.all(np.diff(w, axis=1) <= 1e-6)  # descending gate order
