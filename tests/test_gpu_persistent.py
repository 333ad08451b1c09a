"""The persistent tall gate/up kernel -- one workgroup per compute unit working
through several 192-row tiles, each one's first loads issued under the
previous one's epilogue -- gives the same bits on every run and whatever the
assignment of tiles to workgroups: a layer with more tiles than the machine
has compute units, run twice, and through the separate entry points (one
grouped launch for the routed experts, one for the shared expert, so the
tiles are dealt out differently). Every intermediate is compared, not a
sample. FP8 and MXFP4 weights."""
import numpy as np
import pytest
import torch

from synthetic import LayerConfig
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("precision", ["fp8", "mxfp4"])
def test_persistent_gate_up_repeatable(precision):
    # 1536 tokens, top-4 of 32 experts: ~192 rows per expert, so 192-row
    # tiles on the K = 4096 tall kernels; (32 + 8) M tiles x 8 N tiles of the
    # routed and shared experts, more than 256 compute units take at once
    cfg = LayerConfig(f"persistent_{precision}", 1536, 4096, 32, 4, 1024, 1024, precision,
                      seed=41)
    lt = H.gen(cfg)
    ids, w, y, a = H.run_layer(lt, inter=True)
    rows = np.bincount(ids.reshape(-1), minlength=cfg.E)
    tiles = (int(np.sum(-(-rows // 192))) + -(-cfg.T // 192)) * (cfg.F // 128)
    H.say(f"  rows per expert {rows.min()}..{rows.max()}, ~{tiles} gate/up tiles")
    assert tiles > 256
    _, _, y2, b = H.run_layer(lt, inter=True)
    for key in ("h", "hs", "h_sh", "hs_sh", "eo"):
        assert np.array_equal(a[key], b[key]), f"{key} differs between two runs"
    assert np.array_equal(y, y2), "y differs between two runs"
    st = H.run_stepwise(lt)
    for key in ("h", "hs", "h_sh", "hs_sh", "eo"):
        assert np.array_equal(a[key], st[key]), f"{key} differs from the separate entry points"
    assert np.array_equal(y, st["y"]), "moe_layer_forward differs from the separate entry points"
    assert np.all(np.isfinite(y))
