"""Every HIP kernel of the library compiles for gfx950 without register
spills (no scratch memory per lane): compiled here with hipcc's resource-usage
remarks, the flags the library is built with."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_softmax_amd import build as B

HIPCC = B.hipcc() if shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc") else None


def _usage(src):
    out = os.path.join("/tmp", f"moe_ru_{os.getpid()}_{src}.o")
    r = subprocess.run([HIPCC, *B.FLAGS, "-c", os.path.join(B.SRC, src), "-o", out,
                        "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True)
    if os.path.exists(out):
        os.remove(out)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            kernels[name] = int(m.group(1))
    return kernels


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_no_kernel_spills():
    with cf.ThreadPoolExecutor(max_workers=min(6, len(B.SOURCES))) as ex:
        usage = {}
        for res in ex.map(_usage, B.SOURCES):
            usage.update(res)
    assert len(usage) > 40, "expected every kernel instantiation to be reported"
    spilled = {k: v for k, v in usage.items() if v}
    assert not spilled, f"kernels with scratch memory: {spilled}"
