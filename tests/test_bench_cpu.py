"""bench.py's contract checks that need no GPU: more than one GPU is refused
with a message, and the accounting of algorithmic bytes matches the stated
per-unit figures."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synthetic import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_accounting_per_unit_figures():
    cfg = CONFIGS["decode"]
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[:100] = 1  # 100 touched experts
    a = bench.accounting(cfg, counts)
    d, F, T, k = cfg.d, cfg.F, cfg.T, cfg.k
    w13 = 2 * F * d + 4 * 2 * F     # FP8 codes + one float32 scale per row
    assert a["up_bytes"] == 101 * w13 + (T * k + T) * (d + 4) + T * k * (F + F // 32) + T * (F + F // 32)
    assert a["layer_bytes"] == 101 * (w13 + d * F + 4 * d) + cfg.E * d * 2 + 2 * T * d * 2
    assert a["layer_flops"] == 6.0 * d * (T * k * F + T * F)
    mx = bench.accounting(CONFIGS["decode_mxfp4"], counts)
    w13_mx = 2 * F * d // 2 + 2 * F * d // 32   # E2M1 codes + one E8M0 byte per 32
    assert mx["up_bytes"] - a["up_bytes"] == 101 * (w13_mx - w13)
