"""CPU oracle for the mixture-of-experts layer forward pass.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY. Only `tests/`, the smoke check in
`__graft_entry__.py` and the CPU-baseline leg of `bench.py` may import, call or
run anything in this package. The HIP library (`mixture_experts_softmax_amd`)
never imports it and shares no code, header, table or helper with it.

Contents:
  codecs.py  OCP FP8 E4M3 and bfloat16, written from the formats' definitions.
  moe.py     the layer in float64: router GEMM, softmax, top-k, renormalised
             gates, expert permutation, FP8 activation quantisation, SwiGLU
             expert FFNs, shared expert, combine.
  brute.py   a scalar brute-force loop over all experts for tiny inputs, used to
             pin moe.py.
  qk_rope.py the QK-Norm + RoPE step before attention (per-head RMSNorm, then
             the rotary embedding), in float64.

Parity status: every function is pinned by CPU tests against the formats'
definitions, closed forms, special cases reducing to library routines, and the
brute-force loop. The whole-layer result at the full benchmark sizes has no
published values to compare against; it is pinned only through those checks
on small shapes.
"""
from . import codecs, moe, qk_rope  # noqa: F401
