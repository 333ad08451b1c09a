"""The C ABI library without a GPU: it loads, exports every function that
include/moe.h declares, rejects bad arguments before enqueuing anything, and
its E4M3 encoder (the one the kernels use) agrees with the oracle's codec."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from mixture_experts_softmax_amd import _lib
from oracle import codecs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ["moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward"]:
        assert n in names
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for n in header_functions():
        assert hasattr(L, n), n
    assert _lib.moe_abi_version() == 5


def fp8_shape(**kw):
    p = dict(T=64, d=4096, E=128, k=6, F=1024, F_shared=1024)
    p.update(kw)
    return _lib.shape(p["T"], p["d"], p["E"], p["k"], p["F"], p["F_shared"], "fp8")


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.MOE_OK),
    (dict(T=0), _lib.MOE_OK),
    (dict(T=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=17, E=32), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=9, E=8), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=257), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(d=4000), _lib.MOE_ERR_INVALID_ARG),
    (dict(d=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(F=1000), _lib.MOE_ERR_INVALID_ARG),
    (dict(F_shared=100), _lib.MOE_ERR_INVALID_ARG),
    (dict(F_shared=0), _lib.MOE_OK),
])
def test_check_shape(kw, status):
    assert _lib.moe_check_shape(fp8_shape(**kw)) == status


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 3584, 1 << 22])
@pytest.mark.parametrize("d,E", [(128, 1), (256, 8), (4096, 128), (16384, 256)])
def test_workspace_sizes_for_any_batch(T, d, E):
    """Host-only size queries are defined for every valid shape, the empty
    batch included, and grow with the batch."""
    for prec in ("fp8", "mxfp4", "f32"):
        s = _lib.shape(T, d, E, min(2, E), 128, 128, prec)
        assert _lib.moe_check_shape(s) == _lib.MOE_OK
        lw, rw, pw = (_lib.moe_layer_workspace_size(s), _lib.moe_route_workspace_size(s),
                      _lib.moe_permute_workspace_size(s))
        assert lw >= 0 and rw >= T * E * 4 and pw >= 0
        if T:
            s0 = _lib.shape(T - 1, d, E, min(2, E), 128, 128, prec)
            assert _lib.moe_layer_workspace_size(s0) <= lw


def test_unsupported_dtype_pairs():
    for act, w in [(_lib.MOE_DTYPE_BF16, _lib.MOE_DTYPE_F32), (_lib.MOE_DTYPE_F32, _lib.MOE_DTYPE_FP8_E4M3),
                   (_lib.MOE_DTYPE_FP8_E4M3, _lib.MOE_DTYPE_FP8_E4M3), (7, 2),
                   (_lib.MOE_DTYPE_F32, _lib.MOE_DTYPE_MXFP4), (_lib.MOE_DTYPE_MXFP4, _lib.MOE_DTYPE_MXFP4)]:
        s = _lib.MoeShape(16, 256, 8, 2, 128, 128, act, w)
        assert _lib.moe_check_shape(s) == _lib.MOE_ERR_UNSUPPORTED


def test_mxfp4_shapes_and_workspace():
    """bf16 activations with MXFP4 expert weights form a supported pair whose
    layer workspace equals the FP8 path's (same activation codes and h)."""
    s4 = _lib.shape(64, 4096, 128, 6, 1024, 1024, "mxfp4")
    assert s4.w_dtype == _lib.MOE_DTYPE_MXFP4 and s4.act_dtype == _lib.MOE_DTYPE_BF16
    assert _lib.moe_check_shape(s4) == _lib.MOE_OK
    assert _lib.moe_layer_workspace_size(s4) == _lib.moe_layer_workspace_size(fp8_shape())
    L = _lib.lib()
    A = 1 << 40  # a well-aligned stand-in address; never dereferenced
    need = _lib.moe_layer_workspace_size(s4)
    fake = C.c_void_p(A)
    # scales are required, and (byte arrays) must be 16-byte aligned
    w = _lib.MoeWeights(A, None, A, None, A, A, A, A, A, A)
    assert L.moe_layer_forward(C.byref(s4), C.byref(w), fake, fake, None, None, fake, need, None) == _lib.MOE_ERR_INVALID_ARG
    w = _lib.MoeWeights(A, None, A, A + 1, A, A, A, A, A, A)
    assert L.moe_layer_forward(C.byref(s4), C.byref(w), fake, fake, None, None, fake, need, None) == _lib.MOE_ERR_INVALID_ARG
    f = _lib.MoeFfn(4096, 1024, 128, 384, _lib.MOE_DTYPE_MXFP4, A, None, 6, 64, A, A, A, A, A, A, A)
    f8 = _lib.MoeFfn(4096, 1024, 128, 384, _lib.MOE_DTYPE_FP8_E4M3, A, None, 6, 64, A, A, A, A, A, A, A)
    assert _lib.moe_grouped_ffn_workspace_size(f) == _lib.moe_grouped_ffn_workspace_size(f8)
    odd = _lib.MoeFfn(4096, 1024, 4, 384, _lib.MOE_DTYPE_MXFP4, A, None, 6, 64, A, A, A, A + 4, A, A, A)
    assert L.moe_grouped_ffn(C.byref(odd), fake, 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG


def test_null_pointers_rejected_before_launch():
    L = _lib.lib()
    s = fp8_shape()
    assert L.moe_route_topk(C.byref(s), None, None, None, None, None, None, None, None, None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_combine(C.byref(s), None, None, None, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_permute(C.byref(s), *([None] * 10), 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(C.byref(s), None, None, None, None, None, None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(None, None, None, None, None, None, None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    # T == 0 is a valid no-op even with null pointers
    s0 = fp8_shape(T=0)
    assert L.moe_route_topk(C.byref(s0), None, None, None, None, None, None, None, None, None, 0, None) == _lib.MOE_OK
    assert L.moe_permute(C.byref(s0), *([None] * 10), 0, None) == _lib.MOE_OK
    assert L.moe_layer_forward(C.byref(s0), None, None, None, None, None, None, 0, None) == _lib.MOE_OK


def test_workspace_checks():
    L = _lib.lib()
    s = fp8_shape()
    need = _lib.moe_layer_workspace_size(s)
    assert need > 64 * 6 * 4096 * 2  # holds at least the routed expert outputs
    A = 1 << 40  # a well-aligned stand-in address; never dereferenced
    w = _lib.MoeWeights(A, None, A, A, A, A, A, A, A, A)
    fake = C.c_void_p(1 << 40)
    # missing, short and misaligned workspaces are rejected before any launch
    assert L.moe_layer_forward(C.byref(s), C.byref(w), fake, fake, None, None, None, need, None) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(C.byref(s), C.byref(w), fake, fake, None, None, fake, need - 1, None) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(C.byref(s), C.byref(w), fake, fake, None, None, C.c_void_p((1 << 40) + 16), need, None) == _lib.MOE_ERR_WORKSPACE
    rw = _lib.moe_route_workspace_size(s)
    assert rw >= 64 * 128 * 4
    assert L.moe_route_topk(C.byref(s), fake, fake, None, fake, fake, fake, fake, None, fake, rw - 1, None) == _lib.MOE_ERR_WORKSPACE
    pw = _lib.moe_permute_workspace_size(s)
    assert L.moe_permute(C.byref(s), fake, None, None, fake, fake, fake, None, None, None, fake, pw - 1, None) == _lib.MOE_ERR_WORKSPACE
    # shared expert requested but its weights missing
    w2 = _lib.MoeWeights(A, None, A, A, A, A, None, None, None, None)
    assert L.moe_layer_forward(C.byref(s), C.byref(w2), fake, fake, None, None, fake, need, None) == _lib.MOE_ERR_INVALID_ARG


def test_permute_gather_needs_all_four_pointers():
    """The gather of x into grouped-row order takes xq, x_scale, x_perm and
    x_perm_scale together, on the quantised paths only."""
    L = _lib.lib()
    s = fp8_shape()
    fake = C.c_void_p(1 << 40)
    pw = _lib.moe_permute_workspace_size(s)
    ok = L.moe_permute(C.byref(s), fake, None, None, fake, fake, fake, None, None, None, fake, pw - 1, None)
    assert ok == _lib.MOE_ERR_WORKSPACE  # reaches the workspace check: the pointer set is valid
    for present in ([1, 0, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1], [0, 0, 1, 0]):
        g = [fake if p else None for p in present]
        st = L.moe_permute(C.byref(s), fake, g[0], g[1], fake, fake, fake, g[2], g[3], None, fake, pw, None)
        assert st == _lib.MOE_ERR_INVALID_ARG, present
    s32 = _lib.shape(64, 4096, 128, 6, 1024, 1024, "f32")
    st = L.moe_permute(C.byref(s32), fake, fake, fake, fake, fake, fake, fake, fake, None, fake, 1 << 30, None)
    assert st == _lib.MOE_ERR_INVALID_ARG
    odd = C.c_void_p((1 << 40) + 8)
    st = L.moe_permute(C.byref(s), fake, odd, fake, fake, fake, fake, fake, fake, None, fake, pw, None)
    assert st == _lib.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("prec,Fs", [("fp8", 1024), ("mxfp4", 1024), ("fp8", 0), ("f32", 128)])
@pytest.mark.parametrize("T", [1, 64, 65, 3584])
def test_layer_workspace_regions(prec, Fs, T):
    """The regions of moe_layer_forward's intermediates lie inside its
    workspace, 256-byte aligned, without overlapping, sized as documented."""
    d, E, k, F = (4096, 128, 6, 1024) if prec != "f32" else (256, 8, 2, 128)
    s = _lib.shape(T, d, E, k, F, Fs, prec)
    need = _lib.moe_layer_workspace_size(s)
    r = _lib.moe_layer_workspace_regions(s)
    q = prec != "f32"
    eb = 2 if q else 4
    size = {"xq": T * d, "x_scale": 4 * T, "offsets": 4 * (E + 1), "sorted_pair": 4 * T * k,
            "pair_to_row": 4 * T * k, "h": T * k * F * (1 if q else 4), "h_scale": 4 * T * k * (F // 128),
            "h_shared": T * Fs * (1 if q else 4), "h_shared_scale": 4 * T * (Fs // 128),
            "expert_out": eb * T * k * d, "shared_out": eb * T * d}
    absent = set()
    if not q:
        absent |= {"xq", "x_scale", "h_scale", "h_shared_scale"}
    if not Fs:
        absent |= {"h_shared", "h_shared_scale", "shared_out"}
    spans = []
    for n, off in r.items():
        if n in absent:
            assert off is None, n
            continue
        assert off is not None and off % 256 == 0, n
        assert off + size[n] <= need, n
        spans.append((off, off + size[n], n))
    spans.sort()
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb)
    with pytest.raises(_lib.MoeError):
        _lib.moe_layer_workspace_regions(fp8_shape(k=0))


def test_grouped_ffn_checks():
    L = _lib.lib()
    A = 1 << 40  # a well-aligned stand-in address; never dereferenced
    f = _lib.MoeFfn(4096, 1024, 128, 384, _lib.MOE_DTYPE_FP8_E4M3, A, None, 6, 64, A, A, A, A, A, A, A)
    n = _lib.moe_grouped_ffn_workspace_size(f)
    assert n >= 384 * 1024
    assert L.moe_grouped_ffn(C.byref(f), None, 0, None) == _lib.MOE_ERR_WORKSPACE
    bad = _lib.MoeFfn(4096, 1000, 128, 384, _lib.MOE_DTYPE_FP8_E4M3, 1, None, 6, 64, 1, 1, 1, 1, 1, 1, 1)
    assert L.moe_grouped_ffn(C.byref(bad), None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    nog = _lib.MoeFfn(4096, 1024, 0, 384, _lib.MOE_DTYPE_FP8_E4M3, 1, None, 6, 64, 1, 1, 1, 1, 1, 1, 1)
    assert L.moe_grouped_ffn(C.byref(nog), None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    noscale = _lib.MoeFfn(4096, 1024, 4, 384, _lib.MOE_DTYPE_FP8_E4M3, A, None, 6, 64, A, None, A, A, A, A, A)
    assert L.moe_grouped_ffn(C.byref(noscale), C.c_void_p(1 << 40), 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    misaligned = _lib.MoeFfn(4096, 1024, 4, 384, _lib.MOE_DTYPE_FP8_E4M3, A, None, 6, 64, A + 8, A, A, A, A, A, A)
    assert L.moe_grouped_ffn(C.byref(misaligned), C.c_void_p(1 << 40), 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    f2 = _lib.MoeFfn(4096, 1024, 128, 384, _lib.MOE_DTYPE_FP8_E4M3, A, None, 6, 64, A, A, A, A, A, A, A)
    assert L.moe_grouped_ffn(C.byref(f2), C.c_void_p(A + 128), 1 << 30, None) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_grouped_ffn(C.byref(noscale), C.c_void_p(1 << 40), 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    ub = _lib.MoeFfn(4096, 1024, 4, 384, 1, 1, None, 6, 64, 1, 1, 1, 1, 1, 1, 1)
    assert L.moe_grouped_ffn(C.byref(ub), None, 0, None) == _lib.MOE_ERR_UNSUPPORTED


def test_noalloc_rejects_before_touching_the_device():
    """The no-allocation layer call validates everything on the host: bad
    pointers, and shapes whose workspace exceeds the static scratch, are
    rejected before any HIP call (this container has no GPU)."""
    L = _lib.lib()
    A = 1 << 40  # a well-aligned stand-in address; never dereferenced
    fake = C.c_void_p(A)
    w = _lib.MoeWeights(A, None, A, A, A, A, A, A, A, A)
    s = fp8_shape()
    assert L.moe_layer_forward_noalloc(C.byref(s), None, fake, fake, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(C.byref(s), C.byref(w), None, fake, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(C.byref(s), C.byref(w), C.c_void_p(A + 2), fake, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(C.byref(fp8_shape(k=0)), C.byref(w), fake, fake, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(C.byref(fp8_shape(T=0)), None, None, None, None, None, None) == _lib.MOE_OK
    # the largest batch whose workspace fits, and the first that does not
    fits = [T for T in range(1, 700) if _lib.moe_layer_workspace_size(fp8_shape(T=T)) <= _lib.MOE_NOALLOC_SCRATCH_BYTES]
    assert 288 <= fits[-1] < 699 and fits == list(range(1, fits[-1] + 1))
    big = fp8_shape(T=fits[-1] + 1)
    assert L.moe_layer_forward_noalloc(C.byref(big), C.byref(w), fake, fake, None, None, None) == _lib.MOE_ERR_SCRATCH
    assert L.moe_layer_forward_noalloc(C.byref(fp8_shape(T=3584)), C.byref(w), fake, fake, None, None, None) == _lib.MOE_ERR_SCRATCH
    s100 = _lib.shape(288, 4096, 128, 8, 2048, 2048, "fp8")
    assert _lib.moe_layer_workspace_size(s100) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert "scratch" in _lib.status_string(_lib.MOE_ERR_SCRATCH)


def test_overlap_argument_checks():
    """The second-stream layer call needs its own side stream and two distinct
    events; all checks happen before anything is enqueued."""
    L = _lib.lib()
    A = 1 << 40  # a well-aligned stand-in address; never dereferenced
    fake = C.c_void_p(A)
    w = _lib.MoeWeights(A, None, A, A, A, A, A, A, A, A)
    s = fp8_shape()
    need = _lib.moe_layer_workspace_size(s)
    st, side, e1, e2 = C.c_void_p(A + 256), C.c_void_p(A + 512), C.c_void_p(A + 768), C.c_void_p(A + 1024)
    f = L.moe_layer_forward_overlap
    assert f(C.byref(s), C.byref(w), fake, fake, None, None, fake, need, st, None, e1, e2) == _lib.MOE_ERR_INVALID_ARG
    assert f(C.byref(s), C.byref(w), fake, fake, None, None, fake, need, st, st, e1, e2) == _lib.MOE_ERR_INVALID_ARG
    assert f(C.byref(s), C.byref(w), fake, fake, None, None, fake, need, st, side, None, e2) == _lib.MOE_ERR_INVALID_ARG
    assert f(C.byref(s), C.byref(w), fake, fake, None, None, fake, need, st, side, e1, e1) == _lib.MOE_ERR_INVALID_ARG
    assert f(C.byref(s), C.byref(w), fake, fake, None, None, fake, need - 1, st, side, e1, e2) == _lib.MOE_ERR_WORKSPACE
    assert f(C.byref(s), None, fake, fake, None, None, fake, need, st, side, e1, e2) == _lib.MOE_ERR_INVALID_ARG


def test_status_strings():
    assert _lib.status_string(0) == "ok"
    assert "workspace" in _lib.status_string(-3)
    assert _lib.status_string(123) == "unknown status"


def test_kernel_e4m3_encoder_matches_oracle():
    rng = np.random.default_rng(7)
    pos = codecs.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([
        rng.uniform(-500, 500, 300_000), rng.standard_normal(300_000) * 0.01,
        rng.standard_normal(100_000) * 1e-4, mids, -mids,
        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e4)),
        pos, -pos, [0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30, 2.0 ** -10, 2.0 ** -11],
    ]).astype(np.float32)
    ours = _lib.moe_host_e4m3_encode(v)
    want = codecs.e4m3_encode(v)
    assert np.array_equal(ours, want)


def _qk(**kw):
    p = dict(T=64, n_q=32, n_kv=4, head_dim=128, row_stride=40 * 128, q_offset=0,
             k_offset=32 * 128, eps=1e-6, theta=10000.0, style=_lib.MOE_ROPE_HALVES,
             dtype=_lib.MOE_DTYPE_BF16)
    p.update(kw)
    return _lib.MoeQkShape(p["T"], p["n_q"], p["n_kv"], p["head_dim"], p["row_stride"],
                           p["q_offset"], p["k_offset"], p["eps"], p["theta"], p["style"], p["dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), _lib.MOE_ERR_INVALID_ARG),
    (dict(head_dim=512), _lib.MOE_ERR_INVALID_ARG),
    (dict(n_q=0, n_kv=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(n_q=250, n_kv=7, row_stride=300 * 128), _lib.MOE_ERR_INVALID_ARG),
    (dict(n_q=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(T=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(style=2), _lib.MOE_ERR_INVALID_ARG),
    (dict(eps=-1.0), _lib.MOE_ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.MOE_ERR_INVALID_ARG),
    (dict(theta=0.0), _lib.MOE_ERR_INVALID_ARG),
    (dict(theta=float("inf")), _lib.MOE_ERR_INVALID_ARG),
    (dict(row_stride=40 * 128 + 4), _lib.MOE_ERR_INVALID_ARG),     # not 16-byte rows (bf16)
    (dict(q_offset=4), _lib.MOE_ERR_INVALID_ARG),
    (dict(k_offset=31 * 128), _lib.MOE_ERR_INVALID_ARG),           # overlaps the query heads
    (dict(k_offset=37 * 128), _lib.MOE_ERR_INVALID_ARG),           # runs past the row
    (dict(dtype=_lib.MOE_DTYPE_FP8_E4M3), _lib.MOE_ERR_UNSUPPORTED),
])
def test_qk_norm_rope_rejects_bad_shapes(kw, status):
    """Shape errors are found on the host before anything is enqueued."""
    A = C.c_void_p(1 << 40)  # a well-aligned stand-in address; never dereferenced
    s = _qk(**kw)
    assert _lib.lib().moe_qk_norm_rope(C.byref(s), A, A, A, A, None) == status


def test_qk_norm_rope_pointer_checks():
    L = _lib.lib()
    A = C.c_void_p(1 << 40)
    s = _qk()
    assert L.moe_qk_norm_rope(None, A, A, A, A, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_qk_norm_rope(C.byref(s), None, A, A, A, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_qk_norm_rope(C.byref(s), A, None, A, A, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_qk_norm_rope(C.byref(s), A, A, None, A, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_qk_norm_rope(C.byref(s), A, A, A, C.c_void_p((1 << 40) + 8), None) == _lib.MOE_ERR_INVALID_ARG
    # float32 rows need 4-element (16-byte) alignment only
    s32 = _qk(dtype=_lib.MOE_DTYPE_F32, row_stride=40 * 128 + 4, T=0)
    assert L.moe_qk_norm_rope(C.byref(s32), None, None, None, None, None) == _lib.MOE_OK
    # no key heads: the key weight may be NULL; T == 0 is a no-op
    s0 = _qk(T=0, n_kv=0)
    assert L.moe_qk_norm_rope(C.byref(s0), None, None, None, None, None) == _lib.MOE_OK
