"""The wait counts of the ping-pong gate/up kernel's K loop (csrc/pipeline.h),
compiled here with the host compiler, against a replay of the kernel's load
issue order: for every step count, weight depth and per-step load counts the
kernel can be instantiated with, each count must equal the number of loads
issued after the awaited step's loads up to the point of the wait (too small
a count waits for loads the step does not need; too large a count lets the
step be read before it has landed). Every count also has to fit the 6-bit
vmcnt field."""
import os
import shutil
import subprocess

import pytest

from mixture_experts_softmax_amd import build as B

GXX = shutil.which("g++")

PROGRAM = r"""
#include <cstdio>
#include "pipeline.h"
int main() {
  for (int KT = 2; KT <= 40; ++KT)
    for (int D = 2; D <= 6; ++D) {
      if (D + 1 > KT) continue;
      for (int NA = 1; NA <= 4; ++NA)
        for (int NB = 1; NB <= 4; ++NB)
          for (int kt = 0; kt + 1 < KT; ++kt)
            std::printf("%d %d %d %d %d %d %d\n", KT, D, NA, NB, kt,
                        moe::pp_after_a(kt, D, KT, NA, NB), moe::pp_after_b(kt, D, KT, NA, NB));
    }
  return 0;
}
"""

def _issue_order(KT, D):
    """(kind, step) of every load group in issue order, the position just past
    the prologue, and the position just past LOAD(kt)'s loads for each kt."""
    seq = [("A", 0)] + [("B", s) for s in range(D - 1)] + [("A", 1), ("B", D - 1)]
    pro = len(seq)
    end = []
    for j in range(KT):
        if j + 2 < KT:
            seq.append(("A", j + 2))
        if j + D < KT:
            seq.append(("B", j + D))
        end.append(len(seq))
    return seq, pro, end


def _after(seq, end_pos, item, NA, NB):
    pos = seq.index(item)
    return sum(NA if k == "A" else NB for k, _ in seq[pos + 1:end_pos])


@pytest.mark.skipif(GXX is None, reason="no host C++ compiler")
def test_wait_counts_match_the_issue_order(tmp_path):
    src = tmp_path / "pp.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "pp"
    subprocess.run([GXX, "-std=c++17", "-O1", "-I", B.SRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    rows = [tuple(map(int, line.split())) for line in out.splitlines()]
    assert len(rows) > 10000
    cache = {}
    for KT, D, NA, NB, kt, a, b in rows:
        if (KT, D) not in cache:
            cache[(KT, D)] = _issue_order(KT, D)
        seq, pro, end = cache[(KT, D)]
        # A(kt + 1) is awaited at the start of LOAD(kt), B(kt + 1) at its end
        want_a = _after(seq, end[kt - 1] if kt > 0 else pro, ("A", kt + 1), NA, NB)
        want_b = _after(seq, end[kt], ("B", kt + 1), NA, NB)
        assert (a, b) == (want_a, want_b), (KT, D, NA, NB, kt, a, b, want_a, want_b)


def test_instantiated_counts_fit_vmcnt():
    """The kernel's instantiations (32 K steps, 128-row tiles: four weight
    stages, two activation loads and four (FP8) or two (MXFP4) weight loads
    per thread and step) wait with counts below 64."""
    for D, NA, NB in ((3, 2, 4), (3, 2, 2)):
        seq, pro, end = _issue_order(32, D)
        worst = max(_after(seq, end[kt], ("B", kt + 1), NA, NB) for kt in range(31))
        assert worst < 64
