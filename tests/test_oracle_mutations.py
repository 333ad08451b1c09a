"""Plant plausible mistakes in the oracle (on the CPU) and show that at least one
pin fails for each: the pins are not vacuous."""
import numpy as np
import pytest

from oracle import moe
from tests import oracle_pins


def _any_pin_fails():
    for pin in oracle_pins.ALL:
        try:
            pin()
        except AssertionError:
            return True
    return False


def _swap_gate_up(x, ew):
    F = ew.w13.shape[0] // 2
    w = np.concatenate([ew.w13[F:], ew.w13[:F]])
    return ORIG["ffn_fp32"](x, moe.ExpertWeights(w, ew.w13_scale, ew.w2, ew.w2_scale))


def _no_renorm(p, ids):
    return np.take_along_axis(p, ids.astype(np.int64), axis=1)


def _ties_high_index(l, k):
    T, E = l.shape
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((-np.arange(E), -l[t]))
        out[t] = order[:k]
    return out


def _drop_bias(x, w, bias=None):
    return ORIG["router_logits"](x, w, None)


def _silu_wrong_sign(z):
    return z / (1.0 + np.exp(z))


def _unstable_perm(ids, E):
    P = ORIG["permute"](ids, E)
    sp = P.sorted_pair.copy()
    for e in range(E):
        a, b = P.offsets[e], P.offsets[e + 1]
        sp[a:b] = sp[a:b][::-1]
    p2r = np.empty_like(sp); p2r[sp] = np.arange(sp.size, dtype=sp.dtype)
    return moe.Permutation(P.counts, P.offsets, sp, p2r)


def _quant_scale_255(v):
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.abs(v32).max(axis=-1)
    s = np.where(amax == 0, np.float32(1), (amax / np.float32(255)).astype(np.float32)).astype(np.float32)
    from oracle import codecs
    return codecs.e4m3_encode(v32 / s[..., None]), s


def _w13_scale_by_input(xq, s_x, ew):
    # scale applied along the wrong axis: permute scales across output channels
    return ORIG["ffn_fp8"](xq, s_x, moe.ExpertWeights(ew.w13, ew.w13_scale[::-1].copy(), ew.w2, ew.w2_scale))


def _shared_dropped(w, o_pairs, o_shared):
    return ORIG["combine"](w, o_pairs, None)


def _fp4_high_nibble_first(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0xF
    return out


def _e8m0_bias_126(e):
    return np.ldexp(1.0, np.asarray(e, np.int64) - 126)


def _histogram_tile_63(ids, E, tile=64):
    return ORIG["tile_histogram"](ids, E, 63)


def _gather_slot_not_token(xq, s_x, perm, k):
    tok = perm.sorted_pair.astype(np.int64) % k
    return xq[tok], s_x[tok]


ORIG = {n: getattr(moe, n) for n in
        ["ffn_fp32", "ffn_fp8", "router_logits", "permute", "combine", "tile_histogram"]}

MUTANTS = {
    "swap_gate_up": ("ffn_fp32", _swap_gate_up),
    "no_renormalise": ("gate_weights", _no_renorm),
    "ties_to_high_index": ("topk_ids", _ties_high_index),
    "drop_router_bias": ("router_logits", _drop_bias),
    "silu_wrong_sign": ("silu", _silu_wrong_sign),
    "unstable_group_order": ("permute", _unstable_perm),
    "scale_amax_over_255": ("quantize_rows_e4m3", _quant_scale_255),
    "w13_scale_misindexed": ("ffn_fp8", _w13_scale_by_input),
    "shared_expert_dropped": ("combine", _shared_dropped),
    "fp4_high_nibble_first": ("codecs.unpack_fp4", _fp4_high_nibble_first),
    "e8m0_bias_126": ("codecs.e8m0_decode", _e8m0_bias_126),
    "histogram_tile_63": ("tile_histogram", _histogram_tile_63),
    "gather_slot_not_token": ("gather_rows", _gather_slot_not_token),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr.startswith("codecs."):
        from oracle import codecs
        monkeypatch.setattr(codecs, attr.split(".", 1)[1], fn)
    else:
        monkeypatch.setattr(moe, attr, fn)
    assert _any_pin_fails(), f"no pin catches mutant {name}"
