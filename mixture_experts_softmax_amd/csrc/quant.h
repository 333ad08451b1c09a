// FP8 E4M3 quantisation of bf16 activation rows, one scale per row
// (amax / 448): the x operand of the FP8 expert GEMMs. The pages run those
// GEMMs in FP8 without giving the activations' scaling; a per-token scale is
// the plain reading. Device helpers shared by the launches that quantise x:
// the router's logits launch and, in the layer, the permutation's scan
// launch.
#pragma once

#include "common.h"

namespace moe {

constexpr int kQuantGroup = 8;  // 16-byte loads per lane in flight per group

__device__ inline float absmax8(const v4i& c, float m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)c[q] & 0xffff))));
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)c[q] >> 16))));
  }
  return m;
}

// Eight bf16 values (one 16-byte chunk) divided by s and encoded to E4M3.
// The quotients have magnitude at most 448 (s = amax / 448), where gfx950's
// packed float32 -> FP8 conversion rounds to nearest even and saturates at
// 448 exactly as e4m3_encode does (the two agree bit for bit on every
// float32 of that range, both signs, subnormal results included).
__device__ inline uint2 encode8(const v4i& c, float s) {
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __fdiv_rn(bf16_to_f32((uint16_t)((uint32_t)c[q] & 0xffff)), s);
    f[2 * q + 1] = __fdiv_rn(bf16_to_f32((uint16_t)((uint32_t)c[q] >> 16)), s);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// One wave quantises one bf16 row of length d (a multiple of 8) to FP8 E4M3
// with scale amax/448: an amax pass and an encode pass, each issuing its
// 16-byte loads in groups of 8 per lane (one pass over registers when the
// row is a single group). Loads are unconditional (chunk index
// clamped: a repeated chunk changes no maximum and is never stored) and the
// codes are computed before the guarded stores, so no store waits on a load.
__device__ inline void quantize_row(const uint16_t* __restrict__ xr, int d, int lane,
                                    uint8_t* __restrict__ qr, float* __restrict__ s_out) {
  const int nch = d / 8;  // 8-element chunks in the row
  if (nch <= kWave * kQuantGroup) {
    // the row fits one load group (d <= 4096): it stays in registers between
    // the maximum and the encode, so it is read once
    v4i v[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i)
      v[i] = *reinterpret_cast<const v4i*>(xr + (size_t)min(i * kWave + lane, nch - 1) * 8);
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) am = absmax8(v[i], am);
    am = wave_max(am);
    const float sc = (am > 0.f) ? __fdiv_rn(am, kE4M3Max) : 1.0f;
    uint2 q[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) q[i] = encode8(v[i], sc);
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = i * kWave + lane;
      if (c < nch) *reinterpret_cast<uint2*>(qr + (size_t)c * 8) = q[i];
    }
    if (lane == 0) *s_out = sc;
    return;
  }
  float amax = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kWave * kQuantGroup) {
    v4i v[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = min(c0 + i * kWave + lane, nch - 1);
      v[i] = *reinterpret_cast<const v4i*>(xr + (size_t)c * 8);
    }
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) amax = absmax8(v[i], amax);
  }
  amax = wave_max(amax);
  const float s = (amax > 0.f) ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
  for (int c0 = 0; c0 < nch; c0 += kWave * kQuantGroup) {
    v4i v[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = min(c0 + i * kWave + lane, nch - 1);
      v[i] = *reinterpret_cast<const v4i*>(xr + (size_t)c * 8);
    }
    uint2 q[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) q[i] = encode8(v[i], s);
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = c0 + i * kWave + lane;
      if (c < nch) *reinterpret_cast<uint2*>(qr + (size_t)c * 8) = q[i];
    }
  }
  if (lane == 0) *s_out = s;
}

}  // namespace moe
