"""The library at its size limits, beyond the benchmark's workloads: the
permutation at the largest batch the ABI accepts (T = MOE_MAX_T tokens, the
largest E, 33.5 M pairs, bit-exact against the oracle), routing of a 65,536-token
batch (every id against the oracle), and a 16,384-token layer (its own
permutation bit-exact, outputs against the oracle on sampled tokens)."""
import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib, alloc_workspace
from oracle import inputs as oinputs
from oracle import moe as omoe
from synthetic import CONFIGS
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MAX_T = 1 << 22  # MOE_MAX_T
MAX_E = 256      # MOE_MAX_E


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def test_permute_at_max_tokens():
    """T = MOE_MAX_T, E = 256, k = 8: ids (a_t + j b_t) mod 256 with b_t odd,
    so a token's 8 ids are distinct; 65,536 tiles of 64 tokens."""
    T, E, k = MAX_T, MAX_E, 8
    g = torch.Generator(device=H.DEV).manual_seed(11)
    a = torch.randint(0, E, (T, 1), device=H.DEV, generator=g, dtype=torch.int32)
    b = 2 * torch.randint(0, E // 2, (T, 1), device=H.DEV, generator=g, dtype=torch.int32) + 1
    j = torch.arange(k, device=H.DEV, dtype=torch.int32).view(1, k)
    d_ids = ((a + j * b) % E).to(torch.int32).contiguous()
    s = _lib.shape(T, 128, E, k, 128, 0, "fp8")
    off = torch.empty(E + 1, dtype=torch.int32, device=H.DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    p2r = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    tc = torch.full((T // 64, E), -1, dtype=torch.int32, device=H.DEV)
    ws = alloc_workspace(_lib.moe_permute_workspace_size(s), H.DEV)
    _lib.moe_permute(s, d_ids, off, sp, p2r, ws, tile_counts=tc)
    torch.cuda.synchronize()
    ids = d_ids.cpu().numpy()
    H.say(f"  {T * k} pairs; oracle permutation")
    P = omoe.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), P.offsets)
    assert np.array_equal(sp.cpu().numpy(), P.sorted_pair)
    assert np.array_equal(p2r.cpu().numpy(), P.pair_to_row)
    assert np.array_equal(tc.cpu().numpy(), omoe.tile_histogram(ids, E))


def test_route_topk_65536_tokens():
    cfg = CONFIGS["prefill"].with_(name="route_65536", T=65536, seed=21)
    lt = H.gen(cfg)
    T, k, d = cfg.T, cfg.k, cfg.d
    s = H.shape_of(cfg)
    ids = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
    xq = torch.empty((T, d), dtype=torch.uint8, device=H.DEV)
    xs = torch.empty((T,), dtype=torch.float32, device=H.DEV)
    _lib.moe_route_topk(s, lt.x, lt.w_router, lt.router_bias, ids, w, xq, xs,
                        alloc_workspace(_lib.moe_route_workspace_size(s), H.DEV))
    torch.cuda.synchronize()
    inp = oinputs.layer_inputs(lt)
    x64 = omoe.activations(inp)
    _, _, ids_ref, w_ref = omoe.route(x64, omoe.router_weight(inp), inp.router_bias, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= H.W_MAX_ABS
    rng = np.random.default_rng(cfg.seed)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 254, replace=False)]))
    q_ref, s_ref = omoe.quantize_rows_e4m3(x64[rows])
    assert np.array_equal(xs.cpu().numpy()[rows], s_ref)
    assert np.array_equal(xq.cpu().numpy()[rows], q_ref)


def test_layer_16384_tokens_sampled():
    cfg = CONFIGS["prefill"].with_(name="prefill_16384", T=16384, seed=22)
    lt = H.gen(cfg)
    ids, w, y, mid = H.run_layer(lt, inter=True)
    H.check_routing_invariants(ids, w, cfg.E)
    H.check_permutation(mid, ids, cfg.E)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    H.say(f"  rows per expert: min {counts.min()} max {counts.max()}")
    rng = np.random.default_rng(cfg.seed)
    tok = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 14, replace=False)]))
    inp = oinputs.layer_inputs(lt)
    r_ids, r_w, r_xq, r_sx, r_y64, _ = omoe.layer_forward_tokens(inp, tok)
    assert np.array_equal(ids[tok], r_ids)
    assert np.abs(w[tok] - r_w).max() <= H.W_MAX_ABS
    assert np.array_equal(mid["xq"][tok], r_xq) and np.array_equal(mid["xs"][tok], r_sx)
    bound, _, _, flips = H.fp8_bounds(inp, mid, tokens=tok)
    H.say(f"  h: {flips} validated neighbouring-code decisions on the sampled tokens")
    H.compare_y(y[tok], r_y64, cfg.precision, f"y[{len(tok)} sampled tokens]", bound)
    assert np.all(np.isfinite(y))
