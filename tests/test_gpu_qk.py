"""GPU parity of moe_qk_norm_rope against the float64 oracle, element by
element, at small shapes (both pairings, bf16 and float32, padded rows, one
token, many heads, head_dim 64/128/256, large positions) and at the full
prefill and decode sizes the benchmark times.

Bound per element: the kernel works in float32 (the sines and cosines are
rounded from float64), so before output rounding its value is within
DELTA = 2^-19 (|a| + |b|) of the exact result, where (a, b) is the element's
normalised rotation pair -- about eight float32 roundings of terms of that
size. bf16 output adds half an ulp, at most 2^-8 of the value. Columns
outside the query and key heads must come back bit for bit."""
import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib
from oracle import qk_rope
from synthetic.qk import QK_CONFIGS, QK_PARITY, make_qk, qk_get, values
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

DELTA_REL = 2.0 ** -19
FLIP_MAX = 0.01  # elements whose bf16 rounding differs from the oracle's own


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def run_qk(cfg, qt):
    s = _lib.qk_shape(cfg.T, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.row, cfg.q_offset, cfg.k_offset,
                      cfg.eps, cfg.theta, cfg.style, qt.qkv.dtype)
    out = qt.qkv.clone()
    _lib.moe_qk_norm_rope(s, out, qt.positions, qt.q_weight, qt.k_weight)
    torch.cuda.synchronize()
    return out


def check(cfg, qt, out):
    x = values(qt.qkv)
    args = (qt.positions.cpu().numpy(), values(qt.q_weight), values(qt.k_weight), cfg.n_q,
            cfg.n_kv, cfg.head_dim, cfg.q_offset, cfg.k_offset, cfg.eps, cfg.theta, cfg.style)
    ref = qk_rope.qk_norm_rope(x, *args)
    scale = qk_rope.normalised_pairs(x, *args[1:8], cfg.eps, cfg.style)
    got = values(out)
    touched = np.zeros(cfg.row, bool)
    touched[cfg.q_offset:cfg.q_offset + cfg.n_q * cfg.head_dim] = True
    touched[cfg.k_offset:cfg.k_offset + cfg.n_kv * cfg.head_dim] = True
    assert np.array_equal(got[:, ~touched], x[:, ~touched]), "columns outside q/k changed"
    delta = DELTA_REL * scale[:, touched]
    r = ref[:, touched]
    g = got[:, touched]
    err = np.abs(g - r)
    if cfg.precision == "bf16":
        bound = 2.0 ** -8 * (np.abs(r) + delta) + delta
        ref_b = values(torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16))
        flips = int((g != ref_b).sum())
    else:
        bound = 2.0 ** -24 * np.abs(r) + delta
        flips = 0
    H.say(f"  {cfg.name}: T={cfg.T} heads={cfg.n_q}+{cfg.n_kv} hd={cfg.head_dim} {cfg.style} "
          f"{cfg.precision}: max err {err.max():.3e}, max err/bound "
          f"{np.max(np.divide(err, bound, out=np.zeros_like(err), where=bound > 0)):.3f}, "
          f"{flips} of {g.size} differ from the oracle's own rounding")
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} elements outside their bound"
    assert flips <= FLIP_MAX * g.size + 1


@pytest.mark.parametrize("name", sorted(QK_PARITY) + sorted(QK_CONFIGS))
def test_qk_norm_rope_vs_oracle(name):
    cfg = qk_get(name)
    qt = make_qk(cfg, device=H.DEV)
    check(cfg, qt, run_qk(cfg, qt))


def test_qk_norm_rope_key_heads_only_and_zero_rows():
    """No query heads (the query weight may be NULL), and an all-zero token
    (its heads stay exactly zero: eps keeps the norm finite)."""
    cfg = QK_PARITY["qk_small"].with_(name="qk_k_only", n_q=0)
    qt = make_qk(cfg, device=H.DEV)
    qt.qkv[3].zero_()
    s = _lib.qk_shape(cfg.T, 0, cfg.n_kv, cfg.head_dim, cfg.row, 0, 0, cfg.eps, cfg.theta,
                      cfg.style, qt.qkv.dtype)
    out = qt.qkv.clone()
    _lib.moe_qk_norm_rope(s, out, qt.positions, None, qt.k_weight)
    torch.cuda.synchronize()
    check(cfg, qt, out)
    assert np.all(values(out)[3] == 0)


def test_qk_norm_rope_empty_batch_is_a_no_op():
    cfg = QK_PARITY["qk_small"]
    s = _lib.qk_shape(0, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.row, cfg.q_offset, cfg.k_offset,
                      cfg.eps, cfg.theta, cfg.style, torch.bfloat16)
    _lib.moe_qk_norm_rope(s, None, None, None, None)
    torch.cuda.synchronize()
