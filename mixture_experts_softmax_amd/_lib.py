"""ctypes binding of libmoe.so: the C ABI declared in include/moe.h, with the
same function names. Argument marshalling only: tensors are checked for
device, dtype, contiguity and size (a host pointer or a short buffer handed to
a kernel would fault the GPU), then their device pointers are passed on. All
computation happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH = -5
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20
MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3, MOE_DTYPE_MXFP4 = 0, 1, 2, 3

# Names declared in include/moe.h, in order.
EXPORTS = [
    "moe_abi_version", "moe_status_string", "moe_check_shape",
    "moe_layer_workspace_size", "moe_route_workspace_size", "moe_permute_workspace_size",
    "moe_grouped_ffn_workspace_size", "moe_layer_workspace_regions",
    "moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
    "moe_layer_forward_events", "moe_host_e4m3_encode", "moe_qk_norm_rope",
    "moe_layer_forward_noalloc", "moe_layer_forward_overlap",
]
MOE_ROPE_INTERLEAVED, MOE_ROPE_HALVES = 0, 1


class MoeShape(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("F", C.c_int32), ("F_shared", C.c_int32), ("act_dtype", C.c_int32),
                ("w_dtype", C.c_int32)]


class MoeWeights(C.Structure):
    _fields_ = [("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w13", C.c_void_p), ("w13_scale", C.c_void_p),
                ("w2", C.c_void_p), ("w2_scale", C.c_void_p),
                ("ws13", C.c_void_p), ("ws13_scale", C.c_void_p),
                ("ws2", C.c_void_p), ("ws2_scale", C.c_void_p)]


class MoeFfn(C.Structure):
    _fields_ = [("d", C.c_int32), ("F", C.c_int32), ("num_groups", C.c_int32),
                ("max_rows", C.c_int32), ("w_dtype", C.c_int32),
                ("group_offsets", C.c_void_p), ("row_src", C.c_void_p), ("src_div", C.c_int32),
                ("a_rows", C.c_int32), ("a", C.c_void_p), ("a_scale", C.c_void_p),
                ("w13", C.c_void_p), ("w13_scale", C.c_void_p),
                ("w2", C.c_void_p), ("w2_scale", C.c_void_p), ("out", C.c_void_p),
                ("h_out", C.c_void_p), ("h_scale_out", C.c_void_p)]


class MoeQkShape(C.Structure):
    _fields_ = [("T", C.c_int32), ("n_q", C.c_int32), ("n_kv", C.c_int32),
                ("head_dim", C.c_int32), ("row_stride", C.c_int64), ("q_offset", C.c_int64),
                ("k_offset", C.c_int64), ("eps", C.c_float), ("theta", C.c_float),
                ("style", C.c_int32), ("dtype", C.c_int32)]


MOE_NO_REGION = (1 << 64) - 1
REGIONS = ["xq", "x_scale", "offsets", "sorted_pair", "pair_to_row", "h", "h_scale", "h_shared",
           "h_shared_scale", "expert_out", "shared_out"]


class MoeLayerRegions(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in REGIONS]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixture_experts_softmax_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
        L.moe_abi_version.restype = I32
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [I32]
        L.moe_check_shape.restype = I32
        L.moe_check_shape.argtypes = [P]
        for n in ("moe_layer_workspace_size", "moe_route_workspace_size",
                  "moe_permute_workspace_size", "moe_grouped_ffn_workspace_size"):
            getattr(L, n).restype = I32
            getattr(L, n).argtypes = [P, C.POINTER(SZ)]
        L.moe_layer_workspace_regions.restype = I32
        L.moe_layer_workspace_regions.argtypes = [P, P]
        L.moe_route_topk.restype = I32
        L.moe_route_topk.argtypes = [P] * 10 + [SZ, P]
        L.moe_permute.restype = I32
        L.moe_permute.argtypes = [P] * 11 + [SZ, P]
        L.moe_grouped_ffn.restype = I32
        L.moe_grouped_ffn.argtypes = [P, P, SZ, P]
        L.moe_combine.restype = I32
        L.moe_combine.argtypes = [P] * 7
        L.moe_layer_forward.restype = I32
        L.moe_layer_forward.argtypes = [P, P, P, P, P, P, P, SZ, P]
        L.moe_layer_forward_overlap.restype = I32
        L.moe_layer_forward_overlap.argtypes = [P, P, P, P, P, P, P, SZ, P, P, P, P]
        L.moe_layer_forward_noalloc.restype = I32
        L.moe_layer_forward_noalloc.argtypes = [P] * 7
        L.moe_layer_forward_events.restype = I32
        L.moe_layer_forward_events.argtypes = [P, P, P, P, P, P, P, SZ, P, P, P]
        L.moe_host_e4m3_encode.restype = None
        L.moe_host_e4m3_encode.argtypes = [P, P, C.c_int64]
        L.moe_qk_norm_rope.restype = I32
        L.moe_qk_norm_rope.argtypes = [P] * 6
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


# ------------------------------------------------------------ marshalling --

def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None,
         device: bool = True):
    """Device pointer of a contiguous tensor (None -> NULL) after checks."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, need {numel}")
    return C.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[C.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


_W_DTYPE = {"fp8": MOE_DTYPE_FP8_E4M3, "mxfp4": MOE_DTYPE_MXFP4, "f32": MOE_DTYPE_F32}


def shape(T, d, E, k, F, F_shared, precision: str) -> MoeShape:
    """precision: "fp8" (bf16 activations, E4M3 weights), "mxfp4" (bf16
    activations, MXFP4 weights) or "f32"."""
    if precision not in _W_DTYPE:
        raise ValueError(precision)
    act = MOE_DTYPE_F32 if precision == "f32" else MOE_DTYPE_BF16
    return MoeShape(T, d, E, k, F, F_shared, act, _W_DTYPE[precision])


def _is_fp8(s: MoeShape) -> bool:
    """The quantised path (FP8 activation codes; FP8 or MXFP4 weights)."""
    return s.w_dtype != MOE_DTYPE_F32


def _w_sizes(w_dtype: int, rows: int, cols: int):
    """(weight bytes or elements, scale dtype, scale elements) of a [rows][cols]
    weight matrix: FP8 has one float32 scale per row, MXFP4 packs two codes a
    byte with one E8M0 byte per 32 columns."""
    if w_dtype == MOE_DTYPE_MXFP4:
        return rows * cols // 2, torch.uint8, rows * cols // 32
    return rows * cols, torch.float32, rows


def _act_dtype(s: MoeShape):
    return torch.bfloat16 if _is_fp8(s) else torch.float32


def _w_dtype(s: MoeShape):
    return torch.uint8 if _is_fp8(s) else torch.float32


# ------------------------------------------------------------ the C calls --

def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_check_shape(s: MoeShape) -> int:
    return lib().moe_check_shape(C.byref(s))


def moe_layer_workspace_size(s: MoeShape) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_layer_workspace_size(C.byref(s), C.byref(n)), "moe_layer_workspace_size")
    return n.value


def moe_route_workspace_size(s: MoeShape) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_route_workspace_size(C.byref(s), C.byref(n)), "moe_route_workspace_size")
    return n.value


def moe_permute_workspace_size(s: MoeShape) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_permute_workspace_size(C.byref(s), C.byref(n)), "moe_permute_workspace_size")
    return n.value


def moe_grouped_ffn_workspace_size(f: MoeFfn) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_grouped_ffn_workspace_size(C.byref(f), C.byref(n)),
           "moe_grouped_ffn_workspace_size")
    return n.value


def moe_layer_workspace_regions(s: MoeShape) -> dict:
    """Byte offsets of moe_layer_forward's intermediate results in its
    workspace ({name: offset}; None where the shape has no such result)."""
    r = MoeLayerRegions()
    _check(lib().moe_layer_workspace_regions(C.byref(s), C.byref(r)), "moe_layer_workspace_regions")
    return {n: (None if getattr(r, n) == MOE_NO_REGION else getattr(r, n)) for n in REGIONS}


def moe_route_topk(s: MoeShape, x, w_router, router_bias, topk_ids, topk_w, xq, x_scale,
                   workspace, stream=None, tile_counts=None):
    T, d, E, k = s.T, s.d, s.E, s.k
    fp8 = _is_fp8(s)
    ntiles = (T + 63) // 64
    args = (C.byref(s), _ptr(x, "x", _act_dtype(s), T * d), _ptr(w_router, "w_router", _act_dtype(s), E * d),
            _ptr(router_bias, "router_bias", torch.float32, E),
            _ptr(topk_ids, "topk_ids", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
            _ptr(xq, "xq", torch.uint8, T * d) if fp8 else None,
            _ptr(x_scale, "x_scale", torch.float32, T) if fp8 else None,
            _ptr(tile_counts, "tile_counts", torch.int32, ntiles * E),
            _ptr(workspace, "workspace", torch.uint8),
            workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(lib().moe_route_topk(*args), "moe_route_topk")


def moe_permute(s: MoeShape, topk_ids, offsets, sorted_pair, pair_to_row, workspace, stream=None,
                xq=None, x_scale=None, x_perm=None, x_perm_scale=None, tile_counts=None):
    """Permutation; optionally the gather of xq / x_scale into x_perm /
    x_perm_scale (all four or none) and the per-64-token-tile expert counts."""
    n = s.T * s.k
    ntiles = (s.T + 63) // 64
    _check(lib().moe_permute(C.byref(s), _ptr(topk_ids, "topk_ids", torch.int32, n),
                             _ptr(xq, "xq", torch.uint8, s.T * s.d),
                             _ptr(x_scale, "x_scale", torch.float32, s.T),
                             _ptr(offsets, "offsets", torch.int32, s.E + 1),
                             _ptr(sorted_pair, "sorted_pair", torch.int32, n),
                             _ptr(pair_to_row, "pair_to_row", torch.int32, n),
                             _ptr(x_perm, "x_perm", torch.uint8, n * s.d),
                             _ptr(x_perm_scale, "x_perm_scale", torch.float32, n),
                             _ptr(tile_counts, "tile_counts", torch.int32, ntiles * s.E),
                             _ptr(workspace, "workspace", torch.uint8),
                             workspace.numel() if workspace is not None else 0, _stream(stream)),
           "moe_permute")


def make_ffn(d, F, num_groups, max_rows, fp8, group_offsets, row_src, src_div, a, a_scale,
             w13, w13_scale, w2, w2_scale, out, h_out=None, h_scale_out=None) -> MoeFfn:
    """fp8: True / "fp8" (E4M3 weights), "mxfp4", or False / "f32"."""
    G = num_groups
    fmt = {True: "fp8", False: "f32"}.get(fp8, fp8)
    wdt = _W_DTYPE[fmt]
    fp8 = fmt != "f32"
    wd = torch.uint8 if fp8 else torch.float32
    a_rows = a.shape[0] if a is not None else 0
    n13, sd, ns13 = _w_sizes(wdt, G * 2 * F, d)
    n2, _, ns2 = _w_sizes(wdt, G * d, F)
    return MoeFfn(
        d, F, G, max_rows, wdt,
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(row_src, "row_src", torch.int32, max_rows), src_div, a_rows,
        _ptr(a, "a", wd, a_rows * d),
        _ptr(a_scale, "a_scale", torch.float32, a_rows) if fp8 else None,
        _ptr(w13, "w13", wd, n13),
        _ptr(w13_scale, "w13_scale", sd, ns13) if fp8 else None,
        _ptr(w2, "w2", wd, n2),
        _ptr(w2_scale, "w2_scale", sd, ns2) if fp8 else None,
        _ptr(out, "out", torch.bfloat16 if fp8 else torch.float32, max_rows * d),
        _ptr(h_out, "h_out", wd, max_rows * F),
        _ptr(h_scale_out, "h_scale_out", torch.float32, max_rows * (F // 128)) if fp8 else None)


def moe_grouped_ffn(f: MoeFfn, workspace, stream=None):
    _check(lib().moe_grouped_ffn(C.byref(f), _ptr(workspace, "workspace", torch.uint8),
                                 workspace.numel() if workspace is not None else 0,
                                 _stream(stream)), "moe_grouped_ffn")


def moe_combine(s: MoeShape, expert_out, pair_to_row, topk_w, shared_out, y, stream=None):
    T, d, k = s.T, s.d, s.k
    ad = _act_dtype(s)
    _check(lib().moe_combine(C.byref(s), _ptr(expert_out, "expert_out", ad, T * k * d),
                             _ptr(pair_to_row, "pair_to_row", torch.int32, T * k),
                             _ptr(topk_w, "topk_w", torch.float32, T * k),
                             _ptr(shared_out, "shared_out", ad, T * d),
                             _ptr(y, "y", ad, T * d), _stream(stream)), "moe_combine")


def make_weights(s: MoeShape, w_router, router_bias, w13, w13_scale, w2, w2_scale,
                 ws13=None, ws13_scale=None, ws2=None, ws2_scale=None) -> MoeWeights:
    E, d, F, Fs = s.E, s.d, s.F, s.F_shared
    fp8 = _is_fp8(s)
    wd, ad = _w_dtype(s), _act_dtype(s)
    f32 = torch.float32
    n13, sd, ns13 = _w_sizes(s.w_dtype, E * 2 * F, d)
    n2, _, ns2 = _w_sizes(s.w_dtype, E * d, F)
    nh13, _, nhs13 = _w_sizes(s.w_dtype, 2 * Fs, d)
    nh2, _, nhs2 = _w_sizes(s.w_dtype, d, Fs)
    return MoeWeights(
        _ptr(w_router, "w_router", ad, E * d), _ptr(router_bias, "router_bias", f32, E),
        _ptr(w13, "w13", wd, n13), _ptr(w13_scale, "w13_scale", sd, ns13) if fp8 else None,
        _ptr(w2, "w2", wd, n2), _ptr(w2_scale, "w2_scale", sd, ns2) if fp8 else None,
        _ptr(ws13, "ws13", wd, nh13) if Fs else None,
        _ptr(ws13_scale, "ws13_scale", sd, nhs13) if (Fs and fp8) else None,
        _ptr(ws2, "ws2", wd, nh2) if Fs else None,
        _ptr(ws2_scale, "ws2_scale", sd, nhs2) if (Fs and fp8) else None)


def moe_layer_forward(s: MoeShape, weights: MoeWeights, x, y, topk_ids, topk_w, workspace,
                      stream=None):
    T, d, k = s.T, s.d, s.k
    ad = _act_dtype(s)
    _check(lib().moe_layer_forward(C.byref(s), C.byref(weights), _ptr(x, "x", ad, T * d),
                                   _ptr(y, "y", ad, T * d),
                                   _ptr(topk_ids, "topk_ids", torch.int32, T * k),
                                   _ptr(topk_w, "topk_w", torch.float32, T * k),
                                   _ptr(workspace, "workspace", torch.uint8),
                                   workspace.numel() if workspace is not None else 0,
                                   _stream(stream)), "moe_layer_forward")


def moe_layer_forward_overlap(s: MoeShape, weights: MoeWeights, x, y, topk_ids, topk_w, workspace,
                              side_stream, fork_event: int, join_event: int, stream=None):
    """moe_layer_forward with the shared expert on side_stream (a torch stream),
    forked and joined through two caller-created hipEvent_t handles (int)."""
    T, d, k = s.T, s.d, s.k
    ad = _act_dtype(s)
    _check(lib().moe_layer_forward_overlap(
        C.byref(s), C.byref(weights), _ptr(x, "x", ad, T * d), _ptr(y, "y", ad, T * d),
        _ptr(topk_ids, "topk_ids", torch.int32, T * k), _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel() if workspace is not None else 0,
        _stream(stream), _stream(side_stream), C.c_void_p(fork_event), C.c_void_p(join_event)),
        "moe_layer_forward_overlap")


def moe_layer_forward_noalloc(s: MoeShape, weights: MoeWeights, x, y, topk_ids, topk_w,
                              stream=None):
    """moe_layer_forward with the library's static per-GPU scratch as workspace."""
    T, d, k = s.T, s.d, s.k
    ad = _act_dtype(s)
    _check(lib().moe_layer_forward_noalloc(C.byref(s), C.byref(weights), _ptr(x, "x", ad, T * d),
                                           _ptr(y, "y", ad, T * d),
                                           _ptr(topk_ids, "topk_ids", torch.int32, T * k),
                                           _ptr(topk_w, "topk_w", torch.float32, T * k),
                                           _stream(stream)), "moe_layer_forward_noalloc")


MOE_STEPS = ["route", "permute", "tiles", "gate_up", "down", "combine"]


def moe_layer_forward_events(s: MoeShape, weights: MoeWeights, x, y, topk_ids, topk_w, workspace,
                             start_events, stop_events, stream=None):
    """start_events / stop_events: sequences of len(MOE_STEPS) raw hipEvent_t
    handles (int) or None."""
    T, d, k = s.T, s.d, s.k
    ad = _act_dtype(s)
    n = len(MOE_STEPS)
    arr_t = C.c_void_p * n

    def arr(evs):
        if evs is None:
            return None
        return arr_t(*[C.c_void_p(e) if e else None for e in evs])
    _check(lib().moe_layer_forward_events(C.byref(s), C.byref(weights), _ptr(x, "x", ad, T * d),
                                          _ptr(y, "y", ad, T * d),
                                          _ptr(topk_ids, "topk_ids", torch.int32, T * k),
                                          _ptr(topk_w, "topk_w", torch.float32, T * k),
                                          _ptr(workspace, "workspace", torch.uint8),
                                          workspace.numel() if workspace is not None else 0,
                                          _stream(stream), arr(start_events), arr(stop_events)),
           "moe_layer_forward_events")


def moe_host_e4m3_encode(values) -> "numpy.ndarray":
    import numpy as np
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().moe_host_e4m3_encode(v.ctypes.data, out.ctypes.data, v.size)
    return out


# ------------------------------------------------------- QK-Norm + RoPE --

def qk_shape(T, n_q, n_kv, head_dim, row_stride, q_offset, k_offset, eps, theta, style: str,
             dtype) -> MoeQkShape:
    """style "interleaved" or "halves"; dtype torch.bfloat16 or torch.float32."""
    st = {"interleaved": MOE_ROPE_INTERLEAVED, "halves": MOE_ROPE_HALVES}[style]
    dt = {torch.bfloat16: MOE_DTYPE_BF16, torch.float32: MOE_DTYPE_F32}.get(dtype, -1)
    return MoeQkShape(T, n_q, n_kv, head_dim, row_stride, q_offset, k_offset, eps, theta, st, dt)


def moe_qk_norm_rope(s: MoeQkShape, qkv, positions, q_weight, k_weight, stream=None):
    """In place on qkv [T][row_stride] (contiguous rows of the shape's dtype)."""
    dt = {MOE_DTYPE_BF16: torch.bfloat16, MOE_DTYPE_F32: torch.float32}.get(s.dtype)
    if s.T > 0:
        if qkv is None or qkv.dim() != 2 or qkv.shape[0] < s.T or qkv.shape[1] != s.row_stride:
            raise ValueError("qkv: expected a [T][row_stride] tensor")
    _check(lib().moe_qk_norm_rope(
        C.byref(s), _ptr(qkv, "qkv", dt, s.T * s.row_stride),
        _ptr(positions, "positions", torch.int32, s.T),
        _ptr(q_weight, "q_weight", dt, s.head_dim if s.n_q else 0),
        _ptr(k_weight, "k_weight", dt, s.head_dim if s.n_kv else 0), _stream(stream)),
        "moe_qk_norm_rope")
