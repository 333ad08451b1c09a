"""Full-size workloads on the GPU, in the same launch configuration the
benchmark times (moe_layer_forward on one stream): routing invariants on
every token, and ids / gate weights / outputs against the oracle on sampled
tokens (each token's output depends only on its own row, so the oracle can
compute it alone)."""
import numpy as np
import pytest
import torch

from oracle import inputs as oinputs
from oracle import moe as omoe
from synthetic import CONFIGS
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

SAMPLES = {"decode": 64, "prefill": 16, "b100": 10, "skew": 16, "mixed": 24, "decode_mxfp4": 64,
           "prefill_mxfp4": 16}


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _sample(T, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, T - 1, *extra}
    rest = rng.choice(T, size=min(T, n), replace=False)
    return np.array(sorted(base | set(rest.tolist())))[: max(n, len(base))]


@pytest.mark.parametrize("name", ["decode", "prefill", "b100", "skew", "mixed", "decode_mxfp4",
                                  "prefill_mxfp4"])
def test_fullsize_sampled(name):
    cfg = CONFIGS[name]
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg} redraws={lt.redraws} beta={lt.beta}")
    ids, w, y, mid = H.run_layer(lt, inter=True)
    H.check_routing_invariants(ids, w, cfg.E)
    # the permutation the layer computed, bit-exact against the oracle's
    # stable sort of the layer's ids (every id is checked against the oracle
    # on the sampled tokens below and by the router parity test on all)
    H.check_permutation(mid, ids, cfg.E)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    H.say(f"  touched experts={int((counts > 0).sum())} rows/group max={counts.max()} min={counts.min()}")
    extra = ()
    if cfg.skew:
        assert int((counts[lt.cold] == 0).sum()) == len(lt.cold)
        share = counts[lt.hot].sum() / ids.size
        H.say(f"  hot share={share:.3f}")
        assert 0.45 < share < 0.55
        # tokens landing in the hottest and in the emptiest non-empty group
        hot_e = int(np.argmax(counts))
        extra = tuple(np.nonzero((ids == hot_e).any(1))[0][:3].tolist())
    st = H.run_stepwise(lt)
    assert np.array_equal(st["y"], y), "moe_layer_forward differs from the separate entry points"
    tok = _sample(cfg.T, SAMPLES[name], cfg.seed, extra)
    inp = oinputs.layer_inputs(lt)
    r_ids, r_w, r_xq, r_sx, r_y64, _ = omoe.layer_forward_tokens(inp, tok)
    assert np.array_equal(ids[tok], r_ids)
    assert np.abs(w[tok] - r_w).max() <= H.W_MAX_ABS
    assert np.array_equal(st["xq"][tok], r_xq) and np.array_equal(st["xs"][tok], r_sx)
    assert np.array_equal(mid["xq"][tok], r_xq) and np.array_equal(mid["xs"][tok], r_sx)
    bound, _, _, flips = H.fp8_bounds(inp, mid, tokens=tok)
    H.say(f"  h: {flips} validated neighbouring-code decisions on the sampled tokens")
    H.compare_y(y[tok], r_y64, cfg.precision, f"y[{len(tok)} sampled tokens]", bound)
    assert np.all(np.isfinite(y))


def test_prefill_chunked_equals_whole():
    """The prefill as 14 calls of 256 consecutive tokens gives the same routing
    as one call over all 3584 tokens, and gate weights and outputs equal up to
    the router's float32 summation order (its K split depends on the batch
    size, so logits may differ in the last bits)."""
    cfg = CONFIGS["prefill"]
    lt = H.gen(cfg)
    ids, w, y = H.run_layer(lt)
    L = H.layer(lt)
    yc = torch.empty_like(lt.x)
    idc = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=H.DEV)
    wc = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=H.DEV)
    for c0 in range(0, cfg.T, 256):
        sl = slice(c0, c0 + 256)
        L.forward(lt.x[sl], y=yc[sl], topk_ids=idc[sl], topk_w=wc[sl])
    torch.cuda.synchronize()
    assert np.array_equal(idc.cpu().numpy(), ids)
    dw = np.abs(wc.cpu().numpy() - w).max()
    H.say(f"  chunked vs whole: max |dw| = {dw:.3e}")
    assert dw <= H.W_MAX_ABS
    yc = yc.to(torch.float64).cpu().numpy()
    d = np.abs(yc - y).max()
    H.say(f"  chunked vs whole: max |dy| = {d:.3e} (bit-identical: {d == 0})")
    assert d <= H.FP8_MAX_ABS
