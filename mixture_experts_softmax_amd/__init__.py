"""MI355X-native forward pass of one mixture-of-experts layer (softmax top-k
gating, FP8 or MXFP4 SwiGLU experts, one shared expert) as hand-written HIP kernels for
gfx950 behind a C ABI (include/moe.h, libmoe.so).

This package is the thin Python side: `_lib` mirrors the C entry points one to
one (marshalling only), and `MoELayer` keeps a layer's weights, shape and
workspace together. Every step of the layer runs in the library's kernels; if
the library is missing, importing `_lib` functions raises -- there is no
fallback.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import (MoeError, moe_abi_version, moe_check_shape, moe_combine,  # noqa: F401
                   moe_grouped_ffn, moe_grouped_ffn_workspace_size, moe_layer_forward,
                   moe_layer_workspace_regions, moe_layer_workspace_size, moe_permute,
                   moe_permute_workspace_size,
                   moe_route_topk, moe_host_e4m3_encode, moe_qk_norm_rope, qk_shape)

__all__ = ["MoELayer", "MoeError", "moe_route_topk", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_layer_forward", "moe_qk_norm_rope", "qk_shape"]


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A uint8 device buffer whose start is 256-byte aligned."""
    buf = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 1)]


class MoELayer:
    """One layer: shape, device weights and a reusable workspace.

    precision "fp8": x/y bf16 [T][d], router bf16 [E][d], expert weights uint8
    E4M3 codes with float32 per-output-row scales. precision "mxfp4": as
    "fp8" with MXFP4 expert weights: uint8 w13 [E][2F][d/2] and w2 [E][d][F/2]
    (two E2M1 codes a byte, low nibble first) and uint8 E8M0 scales
    w13_scale [E][2F][d/32], w2_scale [E][d][F/32] (the shared expert alike).
    precision "f32": float32 everywhere, scales None.
    """

    def __init__(self, *, d, E, k, F, F_shared, precision, w_router, router_bias, w13, w13_scale,
                 w2, w2_scale, ws13=None, ws13_scale=None, ws2=None, ws2_scale=None):
        self.d, self.E, self.k, self.F, self.F_shared = d, E, k, F, F_shared
        self.precision = precision
        self.tensors = dict(w_router=w_router, router_bias=router_bias, w13=w13,
                            w13_scale=w13_scale, w2=w2, w2_scale=w2_scale, ws13=ws13,
                            ws13_scale=ws13_scale, ws2=ws2, ws2_scale=ws2_scale)
        self._ws: Optional[torch.Tensor] = None

    def shape(self, T: int) -> _lib.MoeShape:
        return _lib.shape(T, self.d, self.E, self.k, self.F, self.F_shared, self.precision)

    def workspace(self, T: int, device) -> torch.Tensor:
        need = moe_layer_workspace_size(self.shape(T))
        if self._ws is None or self._ws.numel() < need or self._ws.device != torch.device(device):
            self._ws = alloc_workspace(need, device)
        return self._ws

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        T = x.shape[0]
        s = self.shape(T)
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(T, x.device)
        w = _lib.make_weights(s, **self.tensors)
        moe_layer_forward(s, w, x, y, topk_ids, topk_w, ws, stream)
        return y

    def intermediates(self, T: int) -> dict:
        """Views into the workspace of the intermediate results that the last
        forward over T tokens left there (offsets from
        moe_layer_workspace_regions): valid once the stream has reached the end
        of that call, until the next call. Keys: xq, x_scale, offsets,
        sorted_pair, pair_to_row, h, h_scale, h_shared, h_shared_scale,
        expert_out, shared_out (absent where the shape has no such result)."""
        if self._ws is None:
            raise RuntimeError("no forward has run yet")
        s = self.shape(T)
        q = self.precision != "f32"
        E, k, d, F, Fs = self.E, self.k, self.d, self.F, self.F_shared
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        act = torch.bfloat16 if q else f32
        hdt = u8 if q else f32
        layout = {"xq": (u8, (T, d)), "x_scale": (f32, (T,)), "offsets": (i32, (E + 1,)),
                  "sorted_pair": (i32, (T * k,)), "pair_to_row": (i32, (T * k,)),
                  "h": (hdt, (T * k, F)), "h_scale": (f32, (T * k, F // 128)),
                  "h_shared": (hdt, (T, Fs)), "h_shared_scale": (f32, (T, Fs // 128)),
                  "expert_out": (act, (T * k, d)), "shared_out": (act, (T, d))}
        out = {}
        for name, off in moe_layer_workspace_regions(s).items():
            if off is None:
                continue
            dt, shp = layout[name]
            n = 1
            for v in shp:
                n *= v
            nbytes = n * torch.tensor([], dtype=dt).element_size()
            out[name] = self._ws[off:off + nbytes].view(dt).view(shp)
        return out

    __call__ = forward
