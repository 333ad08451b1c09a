"""Seeded synthetic inputs for one MoE layer.

This module only draws random numbers and stores them in the layer's input
formats; it holds none of the layer's arithmetic. Where input selection needs
routing decisions (redrawing tokens whose top-k is a near tie, calibrating the
skew bias) the caller passes those decisions in as `hooks` -- the test suite
passes the CPU oracle's router. Without hooks no token is redrawn and the skew
bias uses a fixed hot-expert boost.

Distributions (the layer's stated workload; the pages give none):
  x        ~ N(0, 1), stored bf16 (FP8 path) or float32
  W_router ~ N(0, 1/sqrt(d)) ([E][d]), stored bf16 or float32
  W13, W2  ~ N(0, 1/sqrt(fan_in)) float32 masters (fan_in = d for W13, F for W2);
             FP8 path: one scale per output row, scale = amax/448, codes =
             E4M3(master / scale) with torch's float8_e4m3fn cast after a clamp
             to +-448; float32 path: the masters themselves.
  skew     8 hot experts get +beta, 40 starved experts get -30 on their logits,
           the rest 0; beta chosen so the hot experts take ~50% of the T*k
           assignments.

Streams: numpy PCG64 children of SeedSequence(seed) for x, the router, the
skew choice and redraws; each expert's weights come from a torch Generator on
the target device seeded from its own child, so experts are generated (and
quantised) one at a time and host memory stays small. Torch's CPU and GPU
generators differ, so the same config drawn on another device holds other
(equally distributed) weights.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Protocol

import numpy as np
import torch

from .configs import LayerConfig

HOT_EXPERTS = 8
COLD_EXPERTS = 40
COLD_BIAS = -30.0
DEFAULT_BETA = 1.5
MIN_TIE_GAP = 1e-5

# child stream indices
_X, _ROUTER, _SKEW, _REDRAW, _SHARED, _EXPERT0 = range(6)


class RoutingHooks(Protocol):
    def near_tie(self, x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
                 k: int, min_gap: float) -> np.ndarray: ...

    def expert_counts(self, x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
                      k: int, E: int) -> np.ndarray: ...


@dataclass
class LayerTensors:
    cfg: LayerConfig
    x: torch.Tensor                   # [T][d] bf16 or f32
    w_router: torch.Tensor            # [E][d] bf16 or f32
    router_bias: Optional[torch.Tensor]  # [E] f32
    w13: torch.Tensor                 # [E][2F][d] uint8 codes or f32
    w13_scale: Optional[torch.Tensor] # [E][2F] f32
    w2: torch.Tensor                  # [E][d][F]
    w2_scale: Optional[torch.Tensor]  # [E][d]
    ws13: Optional[torch.Tensor]      # [2Fs][d]
    ws13_scale: Optional[torch.Tensor]
    ws2: Optional[torch.Tensor]       # [d][Fs]
    ws2_scale: Optional[torch.Tensor]
    redraws: int = 0
    beta: Optional[float] = None
    hot: Optional[np.ndarray] = None
    cold: Optional[np.ndarray] = None


def _children(seed: int, n: int):
    return np.random.SeedSequence(seed).spawn(n)


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _to_act(a: np.ndarray, precision: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if precision != "f32":
        t = t.to(torch.bfloat16)
    return t.to(device)


def act_values(t: torch.Tensor) -> np.ndarray:
    """Stored activations/router weights as float64 numpy (bf16 exact)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def quantize_master_fp8(master: torch.Tensor):
    """Per-output-row FP8 E4M3 storage of a float32 master [rows][cols]:
    returns (uint8 codes, float32 scales)."""
    amax = master.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (master / scale[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


# E2M1 magnitudes in code order, and the midpoints between neighbours.
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def quantize_master_mxfp4(master: torch.Tensor):
    """OCP MXFP4 storage of a float32 master [rows][cols] (cols a multiple of
    32): per 32-column block the shared exponent is floor(log2(amax)) - 2
    (E2M1's largest exponent), the block is divided by 2^exponent and each
    value rounded to the nearest E2M1 value (ties to the even code),
    saturating at 6. Returns (packed codes [rows][cols/2] uint8, element 2i in
    the low nibble; E8M0 scales [rows][cols/32] uint8)."""
    rows, cols = master.shape
    b = master.reshape(rows, cols // 32, 32)
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m 2^ex, 0.5 <= m < 1
    e = torch.where(amax > 0, ex - 1 - 2, torch.full_like(ex, -127)).clamp(-127, 127)
    scaled = b / torch.exp2(e.to(torch.float32))[..., None]
    mag = scaled.abs().clamp(max=6.0)
    mid = torch.tensor(_E2M1_MID, dtype=torch.float32, device=master.device)
    lo = torch.searchsorted(mid, mag.contiguous(), right=False)
    hi = torch.searchsorted(mid, mag.contiguous(), right=True)
    code = torch.where(lo == hi, lo, torch.where(lo % 2 == 0, lo, hi))  # exact midpoint: even code
    code = code.to(torch.uint8) | (torch.signbit(scaled).to(torch.uint8) << 3)
    code = code.reshape(rows, cols)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def _expert(seed_ss, rows13: int, d: int, F: int, precision: str, device):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed_ss))
    m13 = torch.randn(rows13, d, generator=g, device=device, dtype=torch.float32) * (1.0 / math.sqrt(d))
    m2 = torch.randn(d, F, generator=g, device=device, dtype=torch.float32) * (1.0 / math.sqrt(F))
    if precision == "fp8":
        q13, s13 = quantize_master_fp8(m13)
        q2, s2 = quantize_master_fp8(m2)
        return q13, s13, q2, s2
    if precision == "mxfp4":
        q13, s13 = quantize_master_mxfp4(m13)
        q2, s2 = quantize_master_mxfp4(m2)
        return q13, s13, q2, s2
    return m13, None, m2, None


def make_layer(cfg: LayerConfig, device="cpu", hooks: Optional[RoutingHooks] = None,
               min_gap: float = MIN_TIE_GAP, zero_x: bool = False) -> LayerTensors:
    kids = _children(cfg.seed, _EXPERT0 + cfg.E)
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared

    rx = np.random.Generator(np.random.PCG64(kids[_X]))
    x32 = rx.standard_normal((T, d), dtype=np.float32)
    if zero_x:
        x32[:] = 0
    rr = np.random.Generator(np.random.PCG64(kids[_ROUTER]))
    wr32 = (rr.standard_normal((E, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)))

    x_t = _to_act(x32, cfg.precision, "cpu")
    wr_t = _to_act(wr32, cfg.precision, "cpu")
    wr64 = act_values(wr_t)

    bias = None
    beta = hot = cold = None
    if cfg.skew:
        rs = np.random.Generator(np.random.PCG64(kids[_SKEW]))
        order = rs.permutation(E)
        hot, cold = np.sort(order[:HOT_EXPERTS]), np.sort(order[HOT_EXPERTS:HOT_EXPERTS + COLD_EXPERTS])

        def bias_for(b):
            v = np.zeros(E, dtype=np.float32)
            v[cold] = COLD_BIAS
            v[hot] = b
            return v

        beta = DEFAULT_BETA
        if hooks is not None and T > 0:
            x64 = act_values(x_t)
            lo, hi = 0.0, 10.0
            for _ in range(40):  # bisection on the hot share of assignments
                mid = 0.5 * (lo + hi)
                c = hooks.expert_counts(x64, wr64, bias_for(mid), k, E)
                share = c[hot].sum() / float(T * k)
                if share < 0.5:
                    lo = mid
                else:
                    hi = mid
                if abs(share - 0.5) < 0.005:
                    break
            beta = float(np.float32(mid))
        bias = bias_for(beta)

    redraws = 0
    if hooks is not None and T > 0 and not zero_x:  # an all-zero x ties every logit on purpose
        rd = np.random.Generator(np.random.PCG64(kids[_REDRAW]))
        for _ in range(1000):
            bad = hooks.near_tie(act_values(x_t), wr64, bias, k, min_gap)
            n = int(bad.sum())
            if n == 0:
                break
            redraws += n
            x32[bad] = rd.standard_normal((n, d), dtype=np.float32)
            x_t = _to_act(x32, cfg.precision, "cpu")
        else:
            raise RuntimeError("make_layer: near-tie redraw did not converge")

    w13_scale = w2_scale = None
    if cfg.precision == "mxfp4":
        w13 = torch.empty((E, 2 * F, d // 2), dtype=torch.uint8, device=device)
        w2 = torch.empty((E, d, F // 2), dtype=torch.uint8, device=device)
        w13_scale = torch.empty((E, 2 * F, d // 32), dtype=torch.uint8, device=device)
        w2_scale = torch.empty((E, d, F // 32), dtype=torch.uint8, device=device)
    else:
        wdt = torch.uint8 if cfg.precision == "fp8" else torch.float32
        w13 = torch.empty((E, 2 * F, d), dtype=wdt, device=device)
        w2 = torch.empty((E, d, F), dtype=wdt, device=device)
        if cfg.precision == "fp8":
            w13_scale = torch.empty((E, 2 * F), dtype=torch.float32, device=device)
            w2_scale = torch.empty((E, d), dtype=torch.float32, device=device)
    for e in range(E):
        q13, s13, q2, s2 = _expert(kids[_EXPERT0 + e], 2 * F, d, F, cfg.precision, device)
        w13[e].copy_(q13)
        w2[e].copy_(q2)
        if s13 is not None:
            w13_scale[e].copy_(s13)
            w2_scale[e].copy_(s2)
        del q13, q2

    ws13 = ws13_scale = ws2 = ws2_scale = None
    if Fs > 0:
        ws13, ws13_scale, ws2, ws2_scale = _expert(kids[_SHARED], 2 * Fs, d, Fs, cfg.precision, device)

    return LayerTensors(
        cfg=cfg, x=x_t.to(device), w_router=wr_t.to(device),
        router_bias=None if bias is None else torch.from_numpy(bias).to(device),
        w13=w13, w13_scale=w13_scale, w2=w2, w2_scale=w2_scale,
        ws13=ws13, ws13_scale=ws13_scale, ws2=ws2, ws2_scale=ws2_scale,
        redraws=redraws, beta=beta, hot=hot, cold=cold)
