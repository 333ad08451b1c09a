"""moe_layer_forward_noalloc, whose workspace is the library's static per-GPU
scratch, against moe_layer_forward with a caller workspace: bit-identical ids,
gate weights and outputs on two calls in a row (the second with fewer tokens,
so it runs over what the first left in the scratch), a call captured into a
HIP graph replaying bit-identically, and a shape too large for the scratch
rejected with its own status before anything is enqueued."""
import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib
from synthetic import CONFIGS, get
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _both(lt, L, x):
    cfg = lt.cfg
    T = x.shape[0]
    s = L.shape(T)
    W = _lib.make_weights(s, **L.tensors)
    out = []
    for noalloc in (False, True):
        ids = torch.full((T, cfg.k), -1, dtype=torch.int32, device=H.DEV)
        w = torch.full((T, cfg.k), -1.0, dtype=torch.float32, device=H.DEV)
        y = torch.full_like(x, float("nan"))
        if noalloc:
            _lib.moe_layer_forward_noalloc(s, W, x, y, ids, w)
        else:
            _lib.moe_layer_forward(s, W, x, y, ids, w, L.workspace(T, H.DEV))
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), w.cpu().numpy(), y.to(torch.float64).cpu().numpy()))
    return out


@pytest.mark.parametrize("name,second", [("decode", 23), ("fp8_model_m128", 70), ("mx_model_m16", 5)])
def test_noalloc_equals_layer_forward(name, second):
    H.say(f"\n[gpu] noalloc {name}: T={get(name).T} then T={second}")
    cfg = get(name)
    lt = H.gen(cfg)
    L = H.layer(lt)
    for T in (cfg.T, second):
        x = lt.x[:T].contiguous()
        (ia, wa, ya), (ib, wb, yb) = _both(lt, L, x)
        assert np.array_equal(ia, ib), f"T={T}: expert ids differ"
        assert np.array_equal(wa, wb), f"T={T}: gate weights differ"
        assert np.array_equal(ya, yb), f"T={T}: outputs differ"
        assert np.all(np.isfinite(yb))
        H.say(f"  T={T}: ids, weights and y bit-identical")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    cfg = CONFIGS["prefill"]
    s = _lib.shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared, "fp8")
    assert _lib.moe_layer_workspace_size(s) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    A = 1 << 40  # never dereferenced: the call must return before any launch
    W = _lib.MoeWeights(A, None, A, A, A, A, A, A, A, A)
    import ctypes as C
    st = _lib.lib().moe_layer_forward_noalloc(C.byref(s), C.byref(W), C.c_void_p(A), C.c_void_p(A),
                                              None, None, None)
    assert st == _lib.MOE_ERR_SCRATCH


@pytest.mark.parametrize("name", ["decode", "mx_model_m16"])
def test_noalloc_graph_replays_match_layer_forward(name):
    """The callers this entry point is for include code under HIP graph
    capture: after one eager call (which looks up the scratch's device
    address), a captured call replays bit-identically to moe_layer_forward
    with a caller workspace, on three input batches with eager work between
    the replays."""
    H.say(f"\n[gpu] noalloc graph {name}")
    cfg = get(name)
    lt = H.gen(cfg)
    L = H.layer(lt)
    T, k = cfg.T, cfg.k
    s = L.shape(T)
    W = _lib.make_weights(s, **L.tensors)
    x = lt.x.clone()
    y = torch.empty_like(x)
    ids = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        _lib.moe_layer_forward_noalloc(s, W, x, y, ids, w)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        _lib.moe_layer_forward_noalloc(s, W, x, y, ids, w)
    torch.cuda.synchronize()
    perm = torch.from_numpy(np.random.default_rng(9).permutation(T)).to(H.DEV)
    inputs = [lt.x, lt.x[perm].contiguous(), (lt.x.float() * 1.5).to(lt.x.dtype)]
    for rep, xin in enumerate(inputs):
        ye = torch.empty_like(xin)
        ide = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
        we = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
        _lib.moe_layer_forward(s, W, xin, ye, ide, we, L.workspace(T, H.DEV))
        torch.cuda.synchronize()
        x.copy_(xin)
        y.fill_(float("nan"))
        ids.fill_(-1)
        w.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ide), f"replay {rep}: ids differ"
        assert torch.equal(w, we), f"replay {rep}: gate weights differ"
        assert torch.equal(y, ye), f"replay {rep}: outputs differ"
        H.say(f"  replay {rep}: bit-identical to moe_layer_forward")
