"""How fast a weight stream with the tall gate/up kernel's read pattern runs,
by how many bytes each CU keeps in flight (tests/probes/stream_probe.hip):
1,176 tiles of 1 MiB -- the gate/up launch's tile count at T = 3584 -- each
read by one workgroup in 32 steps of 256 rows x 128 bytes, with direct-to-LDS
loads or register loads, 8 or 16 waves, two or three steps ahead. Prints one
line per configuration (the figures behind the tall kernels' design notes) and
asserts only that every configuration runs and streams at a plausible rate."""
import ctypes as C
import os

import pytest
import torch

from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libstream_probe.so")
MIB = 1 << 20
NTILES = 1176
KIB = 1024
CONFIGS = [  # (name, config, LDS bytes per workgroup: 96 KiB or more = one workgroup per CU)
    ("direct-to-LDS, 8 waves, 2 steps ahead", 0, 96 * KIB),
    ("direct-to-LDS, 8 waves, 3 steps ahead", 1, 128 * KIB),
    ("direct-to-LDS, 16 waves, 2 steps ahead", 2, 96 * KIB),
    ("registers, 8 waves, compiler-scheduled", 3, 96 * KIB),
    ("registers, 16 waves, compiler-scheduled", 4, 96 * KIB),
    ("registers then LDS, 8 waves, 2 steps ahead", 5, 96 * KIB),
    ("registers then LDS, 8 waves, 3 steps ahead", 6, 96 * KIB),
    ("registers then LDS, 16 waves, 2 steps ahead", 7, 96 * KIB),
]


def _probe():
    if not os.path.exists(PROBE):
        raise ImportError(f"{PROBE} is missing: build with `python -m mixture_experts_softmax_amd.build`")
    L = C.CDLL(PROBE)
    L.stream_probe.restype = C.c_int
    L.stream_probe.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    return L


def test_weight_stream_rates():
    L = _probe()
    w = torch.zeros(NTILES * MIB, dtype=torch.uint8, device=H.DEV)
    sink = torch.zeros(16, dtype=torch.int32, device=H.DEV)
    st = torch.cuda.current_stream().cuda_stream
    H.say(f"\n  {NTILES} tiles of 1 MiB, 32 steps of 256 rows x 128 B, one workgroup per CU")
    for name, cfg, lds in CONFIGS:
        for _ in range(3):
            assert L.stream_probe(cfg, w.data_ptr(), NTILES, sink.data_ptr(), lds, st) == 0, name
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 20
        a.record()
        for _ in range(n):
            L.stream_probe(cfg, w.data_ptr(), NTILES, sink.data_ptr(), lds, st)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        tbs = NTILES * MIB / us / 1e6
        H.say(f"  {name:46s} {us:7.1f} us  {tbs:5.2f} TB/s")
        assert 1.0 < tbs < 8.0, f"{name}: {tbs:.2f} TB/s is not a plausible HBM rate"
