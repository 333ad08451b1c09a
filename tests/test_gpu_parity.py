"""GPU parity: each C-ABI entry point and the whole layer against the float64
oracle on the same seeded inputs. Integer results (expert ids, permutation,
FP8 codes of x) must be bit-exact; floating point within the stated bounds."""
import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib, alloc_workspace
from oracle import inputs as oinputs
from oracle import moe as omoe
from synthetic import CONFIGS, PARITY, get
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "f32_ragged", "f32_noshared", "fp8_small", "fp8_ragged", "fp8_noshared",
         "fp8_k1", "fp8_kE", "fp8_wide", "fp8_skew_small"]


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", SMALL + ["decode"])
def test_route_topk(name):
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    s = H.shape_of(cfg)
    T, k, d = cfg.T, cfg.k, cfg.d
    ids = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
    fp8 = cfg.precision == "fp8"
    xq = torch.empty((T, d), dtype=torch.uint8, device=H.DEV) if fp8 else None
    xs = torch.empty((T,), dtype=torch.float32, device=H.DEV) if fp8 else None
    _lib.moe_route_topk(s, lt.x, lt.w_router, lt.router_bias, ids, w, xq, xs)
    torch.cuda.synchronize()
    inp = oinputs.layer_inputs(lt)
    x64 = omoe.activations(inp)
    _, _, ids_ref, w_ref = omoe.route(x64, omoe.router_weight(inp), inp.router_bias, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= H.W_MAX_ABS
    if fp8:
        q_ref, s_ref = omoe.quantize_rows_e4m3(x64)
        assert np.array_equal(xs.cpu().numpy(), s_ref)
        assert np.array_equal(xq.cpu().numpy(), q_ref)


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (64, 16, 4), (65, 8, 8), (130, 128, 6),
                                   (1000, 32, 1), (4096, 128, 8), (333, 256, 16)])
def test_permute(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if E > 8:  # leave some experts empty
        ids = np.where(ids == 3, (ids + 1) % E, ids)
        ids = np.stack([row if len(set(row)) == k else rng.permutation([e for e in range(E) if e != 3])[:k]
                        for row in ids]).astype(np.int32)
    s = _lib.shape(T, 128, E, k, 128, 0, "fp8")
    d_ids = torch.from_numpy(ids).to(H.DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=H.DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    p2r = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    ws = alloc_workspace(_lib.moe_permute_workspace_size(s), H.DEV)
    _lib.moe_permute(s, d_ids, off, sp, p2r, ws)
    torch.cuda.synchronize()
    P = omoe.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), P.offsets)
    assert np.array_equal(sp.cpu().numpy(), P.sorted_pair)
    assert np.array_equal(p2r.cpu().numpy(), P.pair_to_row)


def test_permute_out_of_range_ids_get_no_row():
    T, E, k = 10, 8, 2
    ids = np.array([[0, 1]] * T, dtype=np.int32)
    ids[3] = [0, 9]
    ids[7] = [-1, 5]
    s = _lib.shape(T, 128, E, k, 128, 0, "fp8")
    off = torch.empty(E + 1, dtype=torch.int32, device=H.DEV)
    sp = torch.full((T * k,), -7, dtype=torch.int32, device=H.DEV)
    p2r = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    ws = alloc_workspace(_lib.moe_permute_workspace_size(s), H.DEV)
    _lib.moe_permute(s, torch.from_numpy(ids).to(H.DEV), off, sp, p2r, ws)
    torch.cuda.synchronize()
    p2r = p2r.cpu().numpy()
    assert p2r[3 * 2 + 1] == -1 and p2r[7 * 2 + 0] == -1
    assert off.cpu().numpy()[-1] == T * k - 2


@pytest.mark.parametrize("name", ["fp8_small", "fp8_ragged", "fp8_wide", "fp8_skew_small", "tiny",
                                  "f32_ragged"])
def test_grouped_ffn(name):
    """moe_grouped_ffn on the routed groups (oracle routing and x codes as input)."""
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    inp = oinputs.layer_inputs(lt)
    ref = omoe.layer_forward(inp)
    fp8 = cfg.precision == "fp8"
    T, k, d, E, F = cfg.T, cfg.k, cfg.d, cfg.E, cfg.F
    rows = T * k
    off = torch.from_numpy(ref.perm.offsets).to(H.DEV)
    sp = torch.from_numpy(ref.perm.sorted_pair).to(H.DEV)
    if fp8:
        a = torch.from_numpy(ref.xq).to(H.DEV)
        a_s = torch.from_numpy(ref.s_x).to(H.DEV)
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=H.DEV)
    else:
        a = lt.x
        a_s = None
        out = torch.empty((rows, d), dtype=torch.float32, device=H.DEV)
    f = _lib.make_ffn(d, F, E, rows, fp8, off, sp, k, a, a_s, lt.w13, lt.w13_scale, lt.w2,
                      lt.w2_scale, out)
    ws = alloc_workspace(_lib.moe_grouped_ffn_workspace_size(f), H.DEV)
    _lib.moe_grouped_ffn(f, ws)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    H.compare_y(got, ref.expert_out, cfg.precision, "expert_out")
    # the shared expert as one group over all tokens, identity rows
    if cfg.F_shared:
        Fs = cfg.F_shared
        out_s = torch.empty((T, d), dtype=out.dtype, device=H.DEV)
        off_s = torch.tensor([0, T], dtype=torch.int32, device=H.DEV)
        fs = _lib.make_ffn(d, Fs, 1, T, fp8, off_s, None, 1, a, a_s, lt.ws13, lt.ws13_scale, lt.ws2,
                           lt.ws2_scale, out_s)
        ws2 = alloc_workspace(_lib.moe_grouped_ffn_workspace_size(fs), H.DEV)
        _lib.moe_grouped_ffn(fs, ws2)
        torch.cuda.synchronize()
        H.compare_y(out_s.to(torch.float64).cpu().numpy(), ref.shared_out, cfg.precision, "shared_out")


@pytest.mark.parametrize("precision", ["fp8", "f32"])
def test_combine(precision):
    T, d, k, E = 77, 512, 4, 16
    rng = np.random.default_rng(5)
    dt = torch.bfloat16 if precision == "fp8" else torch.float32
    eo = torch.from_numpy(rng.standard_normal((T * k, d)).astype(np.float32)).to(dt)
    so = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dt)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    p2r = rng.permutation(T * k).astype(np.int32)
    s = _lib.shape(T, d, E, k, 128, 128, precision)
    y = torch.empty((T, d), dtype=dt, device=H.DEV)
    _lib.moe_combine(s, eo.to(H.DEV), torch.from_numpy(p2r).to(H.DEV), torch.from_numpy(w).to(H.DEV),
                     so.to(H.DEV), y)
    torch.cuda.synchronize()
    eo64 = eo.to(torch.float64).numpy()
    ref = omoe.combine(w.astype(np.float64), eo64[p2r].reshape(T, k, d), so.to(torch.float64).numpy())
    ref = omoe.round_output(ref, precision)
    got = y.to(torch.float64).cpu().numpy()
    if precision == "fp8":  # within one bf16 rounding of the exact sum
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
    else:
        assert np.abs(got - ref).max() <= 1e-5


@pytest.mark.parametrize("name", SMALL)
def test_layer_forward(name):
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg} redraws={lt.redraws}")
    ids, w, y = H.run_layer(lt)
    ref = omoe.layer_forward(oinputs.layer_inputs(lt))
    assert np.array_equal(ids, ref.ids)
    assert np.abs(w - ref.w).max() <= H.W_MAX_ABS
    H.compare_y(y, ref.y, cfg.precision)


def test_layer_zero_input_gives_zero():
    cfg = get("fp8_small")
    lt = H.gen(cfg, zero_x=True)
    ids, w, y = H.run_layer(lt)
    assert np.all(y == 0)
    assert np.array_equal(ids, np.tile(np.arange(cfg.k), (cfg.T, 1)))


def test_layer_t1_and_empty():
    cfg = get("fp8_ragged")
    lt = H.gen(cfg)
    ids, w, y = H.run_layer(lt, x=lt.x[:1].contiguous())
    inp = oinputs.layer_inputs(lt)
    r_ids, r_w, _, _, _, r_y = omoe.layer_forward_tokens(inp, np.array([0]))
    assert np.array_equal(ids, r_ids)
    H.compare_y(y, r_y, "fp8", "y[T=1]")
    # T == 0: nothing enqueued, output untouched
    y0 = torch.empty((0, cfg.d), dtype=torch.bfloat16, device=H.DEV)
    H.layer(lt).forward(lt.x[:0], y=y0)


def test_layer_deterministic():
    cfg = get("fp8_wide")
    lt = H.gen(cfg)
    a = H.run_layer(lt)
    b = H.run_layer(lt)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
