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
         "fp8_k1", "fp8_kE", "fp8_wide", "fp8_skew_small", "fp8_e256", "fp8_e256_rows",
         "fp8_e256_one_tile", "fp8_e192_one_tile"]
MODEL = ["fp8_model_m16", "fp8_model_m32", "fp8_model_m128", "fp8_model_m192", "fp8_model_f2048",
         "fp8_tall_dpart"]
# MXFP4 expert weights: every kernel variant (tile heights 16 to 192, looped
# and unrolled K loops, resident and looped down GEMMs)
MX = ["mx_small", "mx_ragged", "mx_model_m16", "mx_model_m32", "mx_model_m64", "mx_model_m128",
      "mx_model_m192",
      "mx_model_f2048", "mx_tall_dpart"]


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


# whole-batch routing at the full workload sizes, every token against the
# oracle: the tall-batch logits kernel with 2-chunk (mixed), 4-chunk (prefill,
# skew with its bias and empty experts) and 8-chunk (b100) K slices; d = 640
# takes its looped form
ROUTE_FULL = ["mixed", "prefill", "skew", "b100", "fp8_tall_dpart"]


@pytest.mark.parametrize("name", SMALL + ["decode"] + ROUTE_FULL)
def test_route_topk(name):
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    s = H.shape_of(cfg)
    T, k, d = cfg.T, cfg.k, cfg.d
    ids = torch.empty((T, k), dtype=torch.int32, device=H.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=H.DEV)
    fp8 = cfg.precision != "f32"
    xq = torch.empty((T, d), dtype=torch.uint8, device=H.DEV) if fp8 else None
    xs = torch.empty((T,), dtype=torch.float32, device=H.DEV) if fp8 else None
    tc = torch.full(((T + 63) // 64, cfg.E), -1, dtype=torch.int32, device=H.DEV)
    _lib.moe_route_topk(s, lt.x, lt.w_router, lt.router_bias, ids, w, xq, xs,
                        alloc_workspace(_lib.moe_route_workspace_size(s), H.DEV), tile_counts=tc)
    torch.cuda.synchronize()
    inp = oinputs.layer_inputs(lt)
    x64 = omoe.activations(inp)
    _, _, ids_ref, w_ref = omoe.route(x64, omoe.router_weight(inp), inp.router_bias, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= H.W_MAX_ABS
    assert np.array_equal(tc.cpu().numpy(), omoe.tile_histogram(ids_ref, cfg.E))
    if fp8:
        # FP8 codes of x on every row, or (full-size batches, where the
        # oracle's encoder takes seconds per thousand rows) on 256 sampled
        # rows including the first and the last
        rows = np.arange(T)
        if T > 1024:
            rng = np.random.default_rng(cfg.seed)
            rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 254, replace=False)]))
        q_ref, s_ref = omoe.quantize_rows_e4m3(x64[rows])
        assert np.array_equal(xs.cpu().numpy()[rows], s_ref)
        assert np.array_equal(xq.cpu().numpy()[rows], q_ref)


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (64, 16, 4), (65, 8, 8), (130, 128, 6),
                                   (1000, 32, 1), (4096, 128, 8), (333, 256, 16),
                                   (8200, 128, 6), (2000, 12, 3), (5000, 32, 16),
                                   (256, 64, 16), (257, 64, 16)])
def test_permute(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if E > 8:  # leave some experts empty
        ids = np.where(ids == 3, (ids + 1) % E, ids)
        ids = np.stack([row if len(set(row)) == k else rng.permutation([e for e in range(E) if e != 3])[:k]
                        for row in ids]).astype(np.int32)
    d = 256 if T * k <= 50_000 else 128
    s = _lib.shape(T, d, E, k, 128, 0, "fp8")
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
    # again with the histogram and the gather of (random) x codes and scales
    xq = torch.from_numpy(rng.integers(0, 256, (T, d), dtype=np.uint8)).to(H.DEV)
    xs = torch.from_numpy(rng.uniform(0.01, 3.0, T).astype(np.float32)).to(H.DEV)
    xp = torch.zeros((T * k, d), dtype=torch.uint8, device=H.DEV)
    xps = torch.zeros((T * k,), dtype=torch.float32, device=H.DEV)
    tc = torch.full(((T + 63) // 64, E), -1, dtype=torch.int32, device=H.DEV)
    _lib.moe_permute(s, d_ids, off, sp, p2r, ws, xq=xq, x_scale=xs, x_perm=xp, x_perm_scale=xps,
                     tile_counts=tc)
    torch.cuda.synchronize()
    assert np.array_equal(sp.cpu().numpy(), P.sorted_pair)
    g, gs = omoe.gather_rows(xq.cpu().numpy(), xs.cpu().numpy(), P, k)
    assert np.array_equal(xp.cpu().numpy(), g)
    assert np.array_equal(xps.cpu().numpy(), gs)
    assert np.array_equal(tc.cpu().numpy(), omoe.tile_histogram(ids, E))


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


@pytest.mark.parametrize("name", ["fp8_ragged", "fp8_model_m128", "mx_ragged"])
def test_gathered_rows_feed_grouped_ffn(name):
    """The grouped FFN over rows gathered by moe_permute (row_src = NULL)
    equals, bit for bit, the same call reading x's rows through sorted_pair."""
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    st = H.run_stepwise(lt)
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F
    s = H.shape_of(cfg)
    dev = lambda a: torch.from_numpy(a).to(H.DEV)
    ids, xq, xs = dev(st["ids"]), dev(st["xq"]), dev(st["xs"])
    off = torch.empty(E + 1, dtype=torch.int32, device=H.DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    p2r = torch.empty(T * k, dtype=torch.int32, device=H.DEV)
    xp = torch.empty((T * k, d), dtype=torch.uint8, device=H.DEV)
    xps = torch.empty((T * k,), dtype=torch.float32, device=H.DEV)
    _lib.moe_permute(s, ids, off, sp, p2r, alloc_workspace(_lib.moe_permute_workspace_size(s), H.DEV),
                     xq=xq, x_scale=xs, x_perm=xp, x_perm_scale=xps)
    out = torch.empty((T * k, d), dtype=torch.bfloat16, device=H.DEV)
    f = _lib.make_ffn(d, F, E, T * k, cfg.precision, off, None, 1, xp, xps, lt.w13, lt.w13_scale,
                      lt.w2, lt.w2_scale, out)
    _lib.moe_grouped_ffn(f, alloc_workspace(_lib.moe_grouped_ffn_workspace_size(f), H.DEV))
    torch.cuda.synchronize()
    assert np.array_equal(out.to(torch.float64).cpu().numpy(), st["eo"])


@pytest.mark.parametrize("name", ["fp8_small", "fp8_ragged", "fp8_wide", "fp8_skew_small", "tiny",
                                  "f32_ragged", "fp8_model_m16", "fp8_model_m128", "mx_small",
                                  "mx_ragged", "mx_model_m16", "mx_model_m192"])
def test_grouped_ffn(name):
    """moe_grouped_ffn on the routed groups and on the shared expert, with the
    oracle's routing and x codes as input; h decisions validated, outputs
    within the y bound plus the effect of validated h decisions."""
    from tests import fp8_checks as FC
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg}")
    inp = oinputs.layer_inputs(lt)
    ref = omoe.layer_forward(inp)
    fp8 = cfg.precision != "f32"
    T, k, d, E, F = cfg.T, cfg.k, cfg.d, cfg.E, cfg.F
    rows = T * k
    off = torch.from_numpy(ref.perm.offsets).to(H.DEV)
    sp = torch.from_numpy(ref.perm.sorted_pair).to(H.DEV)
    odt = torch.bfloat16 if fp8 else torch.float32
    hdt = torch.uint8 if fp8 else torch.float32
    if fp8:
        a = torch.from_numpy(ref.xq).to(H.DEV)
        a_s = torch.from_numpy(ref.s_x).to(H.DEV)
    else:
        a, a_s = lt.x, None

    def run(G, offsets, row_src, div, nrows, FF, w13, s13, w2, s2):
        out = torch.empty((nrows, d), dtype=odt, device=H.DEV)
        h = torch.empty((nrows, FF), dtype=hdt, device=H.DEV)
        hs = torch.empty((nrows, FF // 128), dtype=torch.float32, device=H.DEV) if fp8 else None
        f = _lib.make_ffn(d, FF, G, nrows, cfg.precision, offsets, row_src, div, a, a_s, w13, s13, w2,
                          s2, out, h, hs)
        _lib.moe_grouped_ffn(f, alloc_workspace(_lib.moe_grouped_ffn_workspace_size(f), H.DEV))
        torch.cuda.synchronize()
        return (out.to(torch.float64).cpu().numpy(), h.cpu().numpy(),
                None if hs is None else hs.cpu().numpy())

    eo, h, hs = run(E, off, sp, k, rows, F, lt.w13, lt.w13_scale, lt.w2, lt.w2_scale)
    extra = np.zeros_like(eo)
    if fp8:
        flips = 0
        for e in range(E):
            r0, r1 = int(ref.perm.offsets[e]), int(ref.perm.offsets[e + 1])
            if r1 == r0:
                continue
            tok = ref.perm.sorted_pair[r0:r1] // k
            ew = inp.expert(e)
            n, dhq = FC.validate_h(ref.xq[tok], ref.s_x[tok], ew, h[r0:r1], hs[r0:r1])
            flips += n
            extra[r0:r1] = FC.down_effect(dhq, ew)
        H.say(f"  routed h: {flips} validated neighbouring-code decisions of {h.size}")
        FC.check_flip_rate(flips, h.size)
    H.compare_y(eo, ref.expert_out, cfg.precision, "expert_out", extra)
    if cfg.F_shared:
        Fs = cfg.F_shared
        off_s = torch.tensor([0, T], dtype=torch.int32, device=H.DEV)
        so, hsh, hssh = run(1, off_s, None, 1, T, Fs, lt.ws13, lt.ws13_scale, lt.ws2, lt.ws2_scale)
        extra_s = 0.0
        if fp8:
            n, dhq = FC.validate_h(ref.xq, ref.s_x, inp.shared, hsh, hssh)
            H.say(f"  shared h: {n} validated neighbouring-code decisions of {hsh.size}")
            FC.check_flip_rate(n, hsh.size)
            extra_s = FC.down_effect(dhq, inp.shared)
        H.compare_y(so, ref.shared_out, cfg.precision, "shared_out", extra_s)


@pytest.mark.parametrize("precision", ["fp8", "f32"])
def test_combine(precision):
    T, d, k, E = 77, 512, 4, 16
    rng = np.random.default_rng(5)
    dt = torch.bfloat16 if precision != "f32" else torch.float32
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
    pairs = eo64[p2r].reshape(T, k, d)
    so64 = so.to(torch.float64).numpy()
    exact = omoe.combine(w.astype(np.float64), pairs, so64)
    got = y.to(torch.float64).cpu().numpy()
    # float32 accumulation of k+1 terms: <= (k+1) * 2^-24 * sum |terms|
    acc_err = (k + 1) * 2.0 ** -24 * (np.einsum("tj,tjd->td", np.abs(w), np.abs(pairs)) + np.abs(so64))
    if precision != "f32":  # plus half a bf16 ulp (<= 2^-8 relative) for the output rounding
        assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + acc_err * 1.01)
    else:
        assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -24 + acc_err * 1.01)


@pytest.mark.parametrize("name", SMALL + MODEL + MX)
def test_layer_forward(name):
    """moe_layer_forward against the oracle: ids, gate weights, x codes and the
    permutation the layer itself computed (read back from its workspace)
    bit-exact, its own h decisions validated, y within bound; the separate
    entry points give bit-identical results."""
    cfg = get(name)
    lt = H.gen(cfg)
    H.say(f"  cfg={cfg} redraws={lt.redraws}")
    ids, w, y, mid = H.run_layer(lt, inter=True)
    inp = oinputs.layer_inputs(lt)
    ref = omoe.layer_forward(inp)
    assert np.array_equal(ids, ref.ids)
    assert np.abs(w - ref.w).max() <= H.W_MAX_ABS
    H.check_permutation(mid, ref.ids, cfg.E)
    if cfg.precision != "f32":
        assert np.array_equal(mid["xq"], ref.xq) and np.array_equal(mid["xs"], ref.s_x)
    st = H.run_stepwise(lt)
    assert np.array_equal(st["ids"], ids) and np.array_equal(st["w"], w)
    assert np.array_equal(st["y"], y), "moe_layer_forward differs from the separate entry points"
    extra = 0.0
    if cfg.precision != "f32":
        extra, _, _, flips = H.fp8_bounds(inp, mid)
        H.say(f"  h: {flips} validated neighbouring-code decisions")
    else:
        assert np.array_equal(mid["eo"], st["eo"])
    H.compare_y(y, ref.y64, cfg.precision, "y", extra)


def test_layer_zero_input_gives_zero():
    cfg = get("fp8_small")
    lt = H.gen(cfg, zero_x=True)
    ids, w, y = H.run_layer(lt)
    assert np.all(y == 0)
    assert np.array_equal(ids, np.tile(np.arange(cfg.k), (cfg.T, 1)))


def test_layer_t1_and_empty():
    cfg = get("fp8_ragged")
    lt = H.gen(cfg)
    x1 = lt.x[:1].contiguous()
    ids, w, y = H.run_layer(lt, x=x1)
    st = H.run_stepwise(lt, x=x1)
    assert np.array_equal(st["y"], y)
    inp = oinputs.layer_inputs(lt)
    r_ids, r_w, _, _, r_y64, _ = omoe.layer_forward_tokens(inp, np.array([0]))
    assert np.array_equal(ids, r_ids)
    extra, _, _, _ = H.fp8_bounds(inp, st, tokens=np.array([0]))
    H.compare_y(y, r_y64, "fp8", "y[T=1]", extra)
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
