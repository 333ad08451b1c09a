"""The QK-Norm + RoPE input generator: shapes, dtypes, position recipes and
determinism (CPU)."""
import numpy as np
import pytest
import torch

from synthetic.qk import QK_CONFIGS, QK_PARITY, make_qk, values


@pytest.mark.parametrize("name", sorted(QK_PARITY) + ["qk_decode"])
def test_shapes_and_determinism(name):
    cfg = {**QK_PARITY, **QK_CONFIGS}[name]
    a, b = make_qk(cfg), make_qk(cfg)
    assert a.qkv.shape == (cfg.T, (cfg.n_q + 2 * cfg.n_kv) * cfg.head_dim + cfg.pad)
    want = torch.bfloat16 if cfg.precision == "bf16" else torch.float32
    assert a.qkv.dtype == want and a.q_weight.dtype == want and a.positions.dtype == torch.int32
    assert torch.equal(a.qkv, b.qkv) and torch.equal(a.positions, b.positions)
    assert torch.equal(a.q_weight, b.q_weight) and torch.equal(a.k_weight, b.k_weight)
    assert not torch.equal(a.q_weight, a.k_weight)
    p = a.positions.numpy()
    if cfg.pos_mode == "prefill":
        assert np.array_equal(p, np.arange(cfg.T))
    elif cfg.pos_mode == "decode":
        assert p.min() >= 3584 and p.max() < 3584 + 128
    else:
        assert p.min() >= 0 and p.max() < (1 << 20)
    v = values(a.qkv)
    assert abs(v.std() - 1.0) < 0.1 and np.isfinite(v).all()
