// Load counting of the ping-pong gate/up kernel's fully unrolled K loop.
//
// A thread's global loads, in issue order: the prologue issues A(0), B(0) ..
// B(D - 2), A(1), B(D - 1); LOAD(j) issues A(j + 2) then B(j + D), each only
// if that K step exists (KT steps in all). A(s) is the NA activation loads of
// step s, B(s) the NB weight loads of step s, D the weight steps loaded ahead.
// Global loads complete in issue order, so "wait until step s's loads have
// landed" is "wait until at most n loads are outstanding", n the loads issued
// after them so far. These functions give that n for the waits of the K loop;
// the library's CPU tests replay the issue order and check them for every
// step count, depth and load count the kernels instantiate.
//
// Plain constexpr C++: the header compiles under hipcc and under a host-only
// compiler.
#pragma once

#if defined(__HIPCC__)
#define MOE_PP_HD __host__ __device__
#else
#define MOE_PP_HD
#endif

namespace moe {

// #{j in [a, b] : j < c}
MOE_PP_HD constexpr int pp_count_below(int a, int b, int c) {
  return (b < c - 1 ? b : c - 1) - a + 1 > 0 ? (b < c - 1 ? b : c - 1) - a + 1 : 0;
}

// Loads issued after A(kt + 1) by the start of LOAD(kt), before its own
// loads: B(kt - 1 + D), issued with A(kt + 1) in LOAD(kt - 1), or last in the
// prologue when kt = 0 (NA is unused: no activation load follows A(kt + 1)
// before LOAD(kt)).
MOE_PP_HD constexpr int pp_after_a(int kt, int D, int KT, int NA, int NB) {
  static_cast<void>(NA);
  return (kt - 1 + D < KT) ? NB : 0;
}

// Loads issued after B(kt + 1) up to the end of LOAD(kt).
MOE_PP_HD constexpr int pp_after_b(int kt, int D, int KT, int NA, int NB) {
  const int s = kt + 1;
  // loads of the prologue after B(s), when the prologue issued it
  const int pro = (s >= D) ? 0 : (s <= D - 2) ? (D - 2 - s) * NB + NA + NB : 0;
  // LOAD(j) for j in [j0, kt] follow B(s) entirely: A(j + 2) if j + 2 < KT,
  // B(j + D) if j + D < KT
  const int j0 = (s >= D) ? s - D + 1 : 0;
  return pro + NA * pp_count_below(j0, kt, KT - 2) + NB * pp_count_below(j0, kt, KT - D);
}

}  // namespace moe
