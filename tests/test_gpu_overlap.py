"""moe_layer_forward_overlap: the shared expert on a second stream, forked
after the router's logits and joined before the combine, gives results
bit-identical to moe_layer_forward (which the parity tests compare with the
oracle), on the fused decode-sized path and on the scan path of larger
batches; repeated calls stay identical (the streams are properly joined)."""
import ctypes as C

import numpy as np
import pytest
import torch

from mixture_experts_softmax_amd import _lib
from synthetic import get
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _event(hip):
    e = C.c_void_p()
    assert hip.hipEventCreateWithFlags(C.byref(e), 2) == 0  # hipEventDisableTiming
    return e.value


@pytest.mark.parametrize("name", ["fp8_small", "fp8_model_m16", "fp8_model_m128", "fp8_model_m192",
                                  "mx_model_m16", "fp8_noshared", "tiny"])
def test_overlap_equals_single_stream(name):
    cfg = get(name)
    H.say(f"\n[gpu] overlap {name}: {cfg}")
    lt = H.gen(cfg)
    L = H.layer(lt)
    T = cfg.T
    s = L.shape(T)
    W = _lib.make_weights(s, **L.tensors)
    hip = C.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
    hip.hipEventDestroy.argtypes = [C.c_void_p]
    fork, join = _event(hip), _event(hip)
    side = torch.cuda.Stream()
    out = []
    for overlap in (False, True, True):
        ids = torch.full((T, cfg.k), -1, dtype=torch.int32, device=H.DEV)
        w = torch.full((T, cfg.k), -1.0, dtype=torch.float32, device=H.DEV)
        y = torch.full_like(lt.x, float("nan"))
        ws = L.workspace(T, H.DEV)
        if overlap:
            _lib.moe_layer_forward_overlap(s, W, lt.x, y, ids, w, ws, side, fork, join)
        else:
            _lib.moe_layer_forward(s, W, lt.x, y, ids, w, ws)
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), w.cpu().numpy(), y.to(torch.float64).cpu().numpy()))
    for o in out[1:]:
        assert np.array_equal(o[0], out[0][0]) and np.array_equal(o[1], out[0][1])
        assert np.array_equal(o[2], out[0][2]), "outputs differ from moe_layer_forward"
    assert np.all(np.isfinite(out[0][2]))
    hip.hipEventDestroy(C.c_void_p(fork))
    hip.hipEventDestroy(C.c_void_p(join))
