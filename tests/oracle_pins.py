"""Checks that pin the oracle to things other than itself: closed forms,
special cases that reduce to library routines, invariants and a scalar
brute-force loop. Each returns None or raises AssertionError. They are
collected as tests in test_oracle_pins.py and re-run against deliberately
broken copies of the oracle in test_oracle_mutations.py, to show that each
plausible mistake is caught by at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch
import torch.nn.functional as tF

from oracle import brute, codecs, moe


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- routing --

def pin_router_vs_brute():
    rng = _rng(100)
    for T, d, E, k in [(5, 16, 6, 2), (4, 8, 9, 4), (3, 12, 5, 5), (6, 7, 4, 1)]:
        x = rng.standard_normal((T, d))
        w = rng.standard_normal((E, d)) / math.sqrt(d)
        b = rng.standard_normal(E) * 0.5
        _, _, ids, wt = moe.route(x, w, b, k)
        experts = [(np.zeros((2, d)), None, np.zeros((d, 1)), None)] * E
        ids_b, w_b, _ = brute.brute_layer(x, w, b, k, experts, None, fp8=False)
        assert np.array_equal(ids, ids_b)
        assert np.allclose(wt, w_b, atol=1e-14, rtol=0)


def pin_router_k_equals_E_is_softmax():
    rng = _rng(101)
    T, d, E = 7, 10, 6
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    l = x @ w.T
    _, _, ids, wt = moe.route(x, w, None, E)
    full = scipy.special.softmax(l, axis=1)
    assert np.allclose(np.take_along_axis(full, ids.astype(np.int64), 1), wt, atol=1e-15)
    # ids sorted by probability, descending
    assert np.all(np.diff(np.take_along_axis(full, ids.astype(np.int64), 1), axis=1) <= 0)


def pin_router_k1_weight_one():
    rng = _rng(102)
    x = rng.standard_normal((9, 5)); w = rng.standard_normal((7, 5))
    _, _, ids, wt = moe.route(x, w, None, 1)
    assert np.all(wt == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(x @ w.T, axis=1))


def pin_router_all_ties_lowest_index():
    x = np.ones((3, 4)); w = np.zeros((6, 4))
    _, _, ids, wt = moe.route(x, w, None, 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    assert np.allclose(wt, 0.25, atol=1e-15)
    # partial tie: experts 1 and 3 tie for the top, 1 must come first
    w2 = np.zeros((5, 4)); w2[1, 0] = w2[3, 0] = 1.0; w2[4, 0] = 0.5
    _, _, ids2, _ = moe.route(np.array([[1.0, 0, 0, 0]]), w2, None, 3)
    assert list(ids2[0]) == [1, 3, 4]


def pin_router_bias_shifts_logits():
    x = np.array([[1.0, 0.0]]); w = np.array([[0.0, 0.0], [0.0, 0.0], [0.0, 0.0]])
    b = np.array([0.0, math.log(3.0), math.log(2.0)])
    _, p, ids, wt = moe.route(x, w, b, 2)
    assert list(ids[0]) == [1, 2]
    assert np.allclose(p[0], [1 / 6, 3 / 6, 2 / 6], atol=1e-15)
    assert np.allclose(wt[0], [3 / 5, 2 / 5], atol=1e-15)


def pin_router_invariants():
    rng = _rng(103)
    T, d, E, k = 50, 32, 16, 5
    x = rng.standard_normal((T, d)); w = rng.standard_normal((E, d))
    l, _, ids, wt = moe.route(x, w, None, k)
    assert np.allclose(wt.sum(1), 1.0, atol=1e-14)
    for t in range(T):
        assert len(set(ids[t])) == k
        sel = l[t, ids[t]]
        rest = np.delete(l[t], ids[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)


def pin_near_tie_rows():
    l = np.array([[3.0, 2.0, 1.0, 0.0],
                  [3.0, 3.0 - 5e-6, 1.0, 0.0],   # tie inside top-2
                  [3.0, 2.0, 2.0 - 5e-6, 0.0],   # tie at the top-2 boundary
                  [3.0, 2.0, 1.0, 1.0 - 5e-6]])  # tie below the boundary only
    assert list(moe.near_tie_rows(l, 2, 1e-5)) == [False, True, True, False]


# ------------------------------------------------------------ permutation --

def pin_permutation_invariants():
    rng = _rng(104)
    for T, E, k in [(40, 8, 3), (1, 5, 5), (0, 4, 2), (64, 16, 1), (33, 32, 6)]:
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        P = moe.permute(ids, E)
        # counts by explicit loop
        counts = [0] * E
        for t in range(T):
            for j in range(k):
                counts[ids[t, j]] += 1
        assert list(P.counts) == counts
        assert P.offsets[0] == 0 and P.offsets[E] == T * k
        assert np.all(np.diff(P.offsets) == P.counts)
        assert sorted(P.sorted_pair.tolist()) == list(range(T * k))
        for r in range(T * k):
            assert P.pair_to_row[P.sorted_pair[r]] == r
        for e in range(E):
            rows = P.sorted_pair[P.offsets[e]:P.offsets[e + 1]]
            assert all(ids[p // k, p % k] == e for p in rows)
            toks = rows // k
            assert np.all(np.diff(toks) > 0)  # ascending, no token twice


def pin_tile_histogram_by_loop():
    """Per-64-token-tile counts against an explicit loop over tokens and
    slots; summed over tiles they are the permutation's group sizes."""
    rng = _rng(112)
    for T, E, k in [(1, 4, 2), (64, 8, 3), (65, 8, 8), (200, 32, 6), (130, 5, 1)]:
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        H = moe.tile_histogram(ids, E)
        assert H.shape == ((T + 63) // 64, E)
        want = [[0] * E for _ in range((T + 63) // 64)]
        for t in range(T):
            for j in range(k):
                want[t // 64][ids[t, j]] += 1
        assert H.tolist() == want
        assert np.array_equal(H.sum(axis=0), moe.permute(ids, E).counts)
    # out-of-range ids are not counted
    ids = np.array([[0, 9], [-1, 1]], dtype=np.int32)
    assert moe.tile_histogram(ids, 4).tolist() == [[1, 1, 0, 0]]


def pin_gather_rows_by_loop():
    """Grouped rows hold, group by group in ascending token order, the rows of
    the tokens routed to that group (explicit loop over experts and tokens)."""
    rng = _rng(113)
    T, E, k, d = 23, 6, 3, 8
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32)
    xq = rng.integers(0, 256, (T, d), dtype=np.uint8)
    sx = rng.uniform(0.1, 2.0, T).astype(np.float32)
    xp, sp = moe.gather_rows(xq, sx, moe.permute(ids, E), k)
    r = 0
    for e in range(E):
        for t in range(T):
            if e in ids[t]:
                assert np.array_equal(xp[r], xq[t]) and sp[r] == sx[t]
                r += 1
    assert r == T * k


# --------------------------------------------------------------- codecs ---

def pin_quant_rows_exact_and_bounded():
    # a row whose values are already E4M3 values with amax 448: scale 1, exact codes
    vals = codecs.E4M3_TABLE[[0x7E, 0x38, 0x01, 0xB8, 0x00, 0x55]]
    q, s = moe.quantize_rows_e4m3(vals[None, :])
    assert s[0] == 1.0
    assert np.array_equal(codecs.e4m3_decode(q[0]), vals)
    # zero row: scale 1, codes 0
    q0, s0 = moe.quantize_rows_e4m3(np.zeros((1, 8)))
    assert s0[0] == 1.0 and np.all(q0 == 0)
    # random rows: scale = fp32(amax)/448 and the E4M3 rounding bound holds
    rng = _rng(105)
    v = (rng.standard_normal((20, 256)) * rng.uniform(1e-3, 1e3, (20, 1))).astype(np.float32)
    q, s = moe.quantize_rows_e4m3(v)
    amax = np.abs(v).max(1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    y = v.astype(np.float64) / s[:, None].astype(np.float64)
    err = np.abs(codecs.e4m3_decode(q) - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))
    assert np.all(np.abs(codecs.e4m3_decode(q)) <= 448.0)


def pin_quant_blocks_independent():
    h = np.zeros((2, 256), dtype=np.float32)
    h[0, :128] = 1000.0; h[0, 5] = -2000.0
    h[0, 128:] = np.linspace(-1e-3, 1e-3, 128, dtype=np.float32)
    h[1, 200] = 3.0
    q, s = moe.quantize_blocks_e4m3(h)
    assert s.shape == (2, 2)
    assert s[0, 0] == np.float32(2000.0) / np.float32(448.0)
    assert s[0, 1] == np.float32(1e-3) / np.float32(448.0)
    assert s[1, 0] == 1.0 and s[1, 1] == np.float32(3.0) / np.float32(448.0)
    # the small block keeps its precision
    back = codecs.e4m3_decode(q[0, 128:]) * s[0, 1]
    assert np.max(np.abs(back - h[0, 128:])) < 1e-3 * 2 ** -4 * 1.01


# ------------------------------------------------------------------ FFN ---

def _torch_swiglu(x, w1, w3, w2):
    xt = torch.from_numpy(x); a = tF.linear(xt, torch.from_numpy(w1))
    b = tF.linear(xt, torch.from_numpy(w3))
    return tF.linear(tF.silu(a) * b, torch.from_numpy(w2)).numpy()


def pin_dense_swiglu_is_textbook():
    """E = k = 1, no shared expert: the layer is a dense SwiGLU FFN (torch's
    linear + silu in float64)."""
    rng = _rng(106)
    T, d, F = 6, 16, 8
    x = rng.standard_normal((T, d)).astype(np.float32)
    w1 = (rng.standard_normal((F, d)) / 4).astype(np.float32)
    w3 = (rng.standard_normal((F, d)) / 4).astype(np.float32)
    w2 = (rng.standard_normal((d, F)) / 3).astype(np.float32)
    ew = moe.ExpertWeights(np.concatenate([w1, w3]), None, w2, None)
    inp = moe.LayerInputs("f32", x, np.zeros((1, d), np.float32), None, 1, 1, lambda e: ew, None)
    r = moe.layer_forward(inp)
    want = _torch_swiglu(x.astype(np.float64), w1.astype(np.float64), w3.astype(np.float64),
                         w2.astype(np.float64))
    assert np.allclose(r.y64, want, atol=1e-12, rtol=0)


def pin_shared_only_when_routed_zero():
    rng = _rng(107)
    T, d, E, k, F, Fs = 5, 16, 4, 2, 8, 12
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    zero = moe.ExpertWeights(rng.standard_normal((2 * F, d)).astype(np.float32), None,
                             np.zeros((d, F), np.float32), None)
    s1 = (rng.standard_normal((Fs, d)) / 4); s3 = (rng.standard_normal((Fs, d)) / 4)
    s2 = rng.standard_normal((d, Fs)) / 3
    shared = moe.ExpertWeights(np.concatenate([s1, s3]).astype(np.float32), None, s2.astype(np.float32), None)
    inp = moe.LayerInputs("f32", x, wr, None, k, E, lambda e: zero, shared)
    r = moe.layer_forward(inp)
    want = _torch_swiglu(x.astype(np.float64), s1.astype(np.float32).astype(np.float64),
                         s3.astype(np.float32).astype(np.float64), s2.astype(np.float32).astype(np.float64))
    assert np.allclose(r.y64, want, atol=1e-12, rtol=0)


def pin_zero_input_zero_output():
    rng = _rng(108)
    T, d, E, k, F = 3, 128, 4, 2, 128
    x = codecs.bf16_encode(np.zeros((T, d)))
    wr = codecs.bf16_encode(rng.standard_normal((E, d)) / 8)
    ew = moe.ExpertWeights(rng.integers(0, 0x7E, (2 * F, d), dtype=np.uint8),
                           np.full(2 * F, 0.01, np.float32),
                           rng.integers(0, 0x7E, (d, F), dtype=np.uint8), np.full(d, 0.01, np.float32))
    inp = moe.LayerInputs("fp8", x, wr, None, k, E, lambda e: ew, ew)
    r = moe.layer_forward(inp)
    assert np.all(r.y == 0) and np.all(r.s_x == 1.0) and np.all(r.xq == 0)
    assert list(r.ids[0]) == [0, 1]  # all logits 0: lowest indices


def _random_fp8_layer(seed, T, d, E, k, F, Fs, bias=True):
    rng = _rng(seed)
    x = codecs.bf16_encode(rng.standard_normal((T, d)))
    wr = codecs.bf16_encode(rng.standard_normal((E, d)) / math.sqrt(d))
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None

    def mk(F_):
        return moe.ExpertWeights(
            codecs.e4m3_encode(rng.standard_normal((2 * F_, d)) * 40),
            (rng.uniform(0.5, 1.5, 2 * F_) / (40 * math.sqrt(d))).astype(np.float32),
            codecs.e4m3_encode(rng.standard_normal((d, F_)) * 40),
            (rng.uniform(0.5, 1.5, d) / (40 * math.sqrt(F_))).astype(np.float32))
    experts = [mk(F) for _ in range(E)]
    shared = mk(Fs) if Fs else None
    return moe.LayerInputs("fp8", x, wr, b, k, E, lambda e: experts[e], shared), experts, shared


def pin_fp8_layer_vs_brute():
    inp, experts, shared = _random_fp8_layer(109, T=3, d=128, E=4, k=2, F=256, Fs=128)
    r = moe.layer_forward(inp)
    ex = [(e.w13, e.w13_scale, e.w2, e.w2_scale) for e in experts]
    sh = (shared.w13, shared.w13_scale, shared.w2, shared.w2_scale)
    ids, w, y = brute.brute_layer(codecs.bf16_decode(inp.x), codecs.bf16_decode(inp.w_router),
                                  inp.router_bias, inp.k, ex, sh, fp8=True)
    assert np.array_equal(r.ids, ids)
    assert np.allclose(r.w, w, atol=1e-14)
    assert np.allclose(r.y64, y, atol=1e-9, rtol=0)


def pin_f32_layer_vs_brute():
    rng = _rng(110)
    T, d, E, k, F, Fs = 4, 12, 5, 3, 6, 4
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / 3).astype(np.float32)
    b = (rng.standard_normal(E) * 0.2).astype(np.float32)

    def mk(F_):
        return moe.ExpertWeights((rng.standard_normal((2 * F_, d)) / 3).astype(np.float32), None,
                                 (rng.standard_normal((d, F_)) / 2).astype(np.float32), None)
    experts = [mk(F) for _ in range(E)]
    shared = mk(Fs)
    inp = moe.LayerInputs("f32", x, wr, b, k, E, lambda e: experts[e], shared)
    r = moe.layer_forward(inp)
    ids, w, y = brute.brute_layer(x.astype(np.float64), wr.astype(np.float64), b, k,
                                  [(e.w13, None, e.w2, None) for e in experts],
                                  (shared.w13, None, shared.w2, None), fp8=False)
    assert np.array_equal(r.ids, ids)
    assert np.allclose(r.y64, y, atol=1e-12, rtol=0)


def _random_mx_layer(seed, T, d, E, k, F, Fs):
    rng = _rng(seed)
    x = codecs.bf16_encode(rng.standard_normal((T, d)))
    wr = codecs.bf16_encode(rng.standard_normal((E, d)) / math.sqrt(d))

    def mk(F_):
        # random nibbles, block exponents around 2^-7 (weights of order 0.01-0.05)
        return moe.ExpertWeights(
            rng.integers(0, 256, (2 * F_, d // 2), dtype=np.uint8),
            rng.integers(118, 123, (2 * F_, d // 32), dtype=np.uint8),
            rng.integers(0, 256, (d, F_ // 2), dtype=np.uint8),
            rng.integers(118, 123, (d, F_ // 32), dtype=np.uint8), "mxfp4")
    experts = [mk(F) for _ in range(E)]
    shared = mk(Fs) if Fs else None
    return moe.LayerInputs("mxfp4", x, wr, None, k, E, lambda e: experts[e], shared), experts, shared


def pin_mxfp4_layer_vs_brute():
    """MXFP4 expert weights: the layer equals the scalar loop that unpacks
    each nibble and applies its block's power of two itself."""
    inp, experts, shared = _random_mx_layer(112, T=3, d=128, E=4, k=2, F=256, Fs=128)
    r = moe.layer_forward(inp)
    ex = [(e.w13, e.w13_scale, e.w2, e.w2_scale) for e in experts]
    sh = (shared.w13, shared.w13_scale, shared.w2, shared.w2_scale)
    ids, w, y = brute.brute_layer(codecs.bf16_decode(inp.x), codecs.bf16_decode(inp.w_router),
                                  None, inp.k, ex, sh, fp8=True, mxfp4=True)
    assert np.array_equal(r.ids, ids)
    assert np.allclose(r.y64, y, atol=1e-9, rtol=0)


def pin_mxfp4_decode_worked_example():
    """One row, two blocks: byte 0x21 holds element 0 = 0.5 (code 1, low
    nibble) and element 1 = 1.0 (code 2); block 0 scale 2^3, block 1 scale
    2^-1; byte 0xF7 holds 6.0 (code 7) then -6.0 (code 0xF)."""
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 16] = 0xF7            # element 32: 6.0, element 33: -6.0
    scales = np.array([[127 + 3, 127 - 1]], np.uint8)
    v = codecs.mxfp4_decode(packed, scales)
    assert v.shape == (1, 64)
    assert v[0, 0] == 4.0 and v[0, 1] == 8.0 and np.all(v[0, 2:32] == 0)
    assert v[0, 32] == 3.0 and v[0, 33] == -3.0 and np.all(v[0, 34:] == 0)


def pin_mxfp4_dense_is_textbook():
    """E = k = 1 with MXFP4 weights: the layer is torch's SwiGLU on the
    decoded weights and the quantised activations, with h quantised per
    128-column block."""
    inp, experts, _ = _random_mx_layer(113, T=4, d=128, E=1, k=1, F=128, Fs=0)
    r = moe.layer_forward(inp)
    ew = experts[0]
    w13 = codecs.mxfp4_decode(ew.w13, ew.w13_scale)
    w2 = codecs.mxfp4_decode(ew.w2, ew.w2_scale)
    xq = codecs.e4m3_decode(r.xq) * r.s_x.astype(np.float64)[:, None]
    gu = tF.linear(torch.from_numpy(xq), torch.from_numpy(w13))
    h = (tF.silu(gu[:, :128]) * gu[:, 128:]).numpy()
    hq, s_h = moe.quantize_blocks_e4m3(h)
    want = tF.linear(torch.from_numpy(codecs.e4m3_decode(hq) * s_h.astype(np.float64)),
                     torch.from_numpy(w2)).numpy()
    assert np.allclose(r.y64, want, atol=1e-10, rtol=0)


def pin_worked_example_closed_form():
    """Hand-derived layer: d=2, E=3, top-2, F=1, one shared expert.
    logits [ln4, 0, ln2] -> p = [4, 1, 2]/7 -> ids [0, 2], w = [2/3, 1/3];
    expert 0: g = x0 = 1, u = x1 = 2, h = 2 silu(1), o = [h, 0];
    expert 2: g = 0 -> h = 0; shared: g = x1 = 2, u = x0 = 1, o_s = [0, silu(2)]."""
    x = np.array([[1.0, 2.0]], np.float32)
    wr = np.array([[math.log(4.0), 0], [0, 0], [0, math.log(2.0) / 2]], np.float32)
    e0 = moe.ExpertWeights(np.array([[1, 0], [0, 1]], np.float32), None, np.array([[1], [0]], np.float32), None)
    e1 = moe.ExpertWeights(np.array([[5, 5], [5, 5]], np.float32), None, np.array([[7], [7]], np.float32), None)
    e2 = moe.ExpertWeights(np.array([[0, 0], [3, 1]], np.float32), None, np.array([[9], [4]], np.float32), None)
    sh = moe.ExpertWeights(np.array([[0, 1], [1, 0]], np.float32), None, np.array([[0], [1]], np.float32), None)
    inp = moe.LayerInputs("f32", x, wr, None, 2, 3, lambda e: [e0, e1, e2][e], sh)
    r = moe.layer_forward(inp)
    assert list(r.ids[0]) == [0, 2]
    assert np.allclose(r.w[0], [2 / 3, 1 / 3], atol=1e-7)
    silu = lambda z: z / (1 + math.exp(-z))
    assert np.allclose(r.y64[0], [2 / 3 * 2 * silu(1.0), silu(2.0)], atol=1e-7)


def pin_token_subset_matches_full():
    inp, _, _ = _random_fp8_layer(111, T=9, d=128, E=6, k=3, F=128, Fs=128)
    full = moe.layer_forward(inp)
    tok = np.array([0, 4, 8, 5])
    ids, w, xq, sx, y64, y = moe.layer_forward_tokens(inp, tok)
    assert np.array_equal(ids, full.ids[tok]) and np.array_equal(w, full.w[tok])
    assert np.array_equal(xq, full.xq[tok]) and np.array_equal(sx, full.s_x[tok])
    assert np.allclose(y64, full.y64[tok], atol=1e-12, rtol=0)


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
