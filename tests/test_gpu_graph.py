"""The layer captured into a HIP graph (torch.cuda.CUDAGraph on the capturing
stream) and replayed: every replay, with eager work and synchronisations in
between and new inputs copied into the captured buffers, gives the eager
call's ids, gate weights and outputs bit for bit. The library enqueues only
kernels (no memset, copy, allocation or synchronisation), so the whole chain
is capturable."""
import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib
from synthetic import CONFIGS, get
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["decode", "decode_mxfp4", "fp8_ragged", "tiny"])
def test_graph_replays_match_eager(name):
    cfg = CONFIGS[name] if name in CONFIGS else get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    L = H.layer(lt)
    T, k = cfg.T, cfg.k
    s = L.shape(T)
    ws = L.workspace(T, H.DEV)
    W = _lib.make_weights(s, **L.tensors)
    x = lt.x.clone()
    y = torch.empty_like(x)
    ids = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=H.DEV)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        _lib.moe_layer_forward(s, W, x, y, ids, w, ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        _lib.moe_layer_forward(s, W, x, y, ids, w, ws)
    torch.cuda.synchronize()

    # three input batches: the generated one, a permutation of its rows, and
    # a rescaled copy (different routing and quantisation scales)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(T)).to(H.DEV)
    inputs = [lt.x, lt.x[perm].contiguous(), (lt.x.float() * 1.75).to(lt.x.dtype)]
    for rep, xin in enumerate(inputs):
        # eager reference on separate buffers
        ye = torch.empty_like(xin)
        ide = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
        we = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
        L.forward(xin, y=ye, topk_ids=ide, topk_w=we)
        torch.cuda.synchronize()
        # replay on the captured buffers, after poisoning the outputs
        x.copy_(xin)
        y.fill_(float("nan"))
        ids.fill_(-1)
        w.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ide), f"replay {rep}: ids differ"
        assert torch.equal(w, we), f"replay {rep}: gate weights differ"
        assert torch.equal(y, ye), f"replay {rep}: outputs differ"
        H.say(f"  replay {rep}: bit-identical to the eager call")
