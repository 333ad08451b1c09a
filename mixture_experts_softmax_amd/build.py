"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m mixture_experts_softmax_amd.build [--verbose]
Objects go to _build/ at the repository root; the library is written next to
this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "route.hip", "permute.hip", "ffn.hip", "combine.hip", "qk_rope.hip"]
# test-only device probes (tests/probes/<name>.hip -> tests/probes/lib<name>.so)
PROBES = ["mfma_fp8_probe", "stream_probe"]
PROBE_DIR = os.path.join(ROOT, "tests", "probes")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # keep the compiler from emitting packed float32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INC, "-I", SRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compiles every source and links libmoe.so. Always rebuilds."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_run, [cc, *FLAGS, "-c", os.path.join(SRC, src), "-o", obj], verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    build_probes(verbose)
    return LIB


def build_probes(verbose: bool = False):
    """Compiles the test suite's device probes (not part of libmoe)."""
    cc = hipcc()
    for name in PROBES:
        src = os.path.join(PROBE_DIR, name + ".hip")
        if not os.path.exists(src):
            continue
        out = os.path.join(PROBE_DIR, "lib" + name + ".so")
        _run([cc, *FLAGS, "-shared", src, "-o", out + ".tmp"], verbose)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
