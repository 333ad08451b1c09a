// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// Number formats.
// ---------------------------------------------------------------------------

// float32 -> OCP E4M3 code: round to nearest even, saturate at +-448, keep the
// sign (so a negative value that rounds to zero gives 0x80).
__host__ __device__ inline uint8_t e4m3_encode(float v) {
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  float a;
  __builtin_memcpy(&a, &ua, 4);
  if (!(a < kE4M3Max)) return (uint8_t)(sign | 0x7Eu);
  if (a >= 0.015625f) {  // normal E4M3 range: keep 3 of the 23 mantissa bits
    const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
    const uint32_t e = (r >> 23) - 120u;  // (e32 - 127) + 7
    const uint32_t m = (r >> 20) & 7u;
    return (uint8_t)(sign | (e << 3) | m);
  }
  // subnormal E4M3: multiples of 2^-9; a * 512 is exact, rint rounds half to even
  const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);
  return (uint8_t)(sign | m);
}

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bf16, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Two float32 -> two bf16 in one dword (a low, b high) by gfx950's packed
// conversion (v_cvt_pk_bf16_f32), which rounds to nearest even: the same
// bits as f32_to_bf16 for finite inputs, in one instruction.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes).
// ---------------------------------------------------------------------------

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// max over the 16 lanes that share (lane / 16)
__device__ inline float max16(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// Matrix cores. D = A * B + C on a 16x16 tile.
//   A operand: lane l holds row (l % 16) of A, B operand: lane l holds column
//   (l % 16) of B; both hold the same K slice, chosen by (l / 16) and the
//   register position, so any consistent K placement gives A * B.
//   Result: lane l, element q holds D[4 * (l / 16) + q][l % 16].
// ---------------------------------------------------------------------------

// FP8 E4M3 x FP8 E4M3, K = 128 (32 bytes per lane). Scale operands 0 select
// the unscaled instruction.
__device__ inline v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 x bf16, K = 32 (8 values per lane).
__device__ inline v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer store resource over [base, base + bytes): a lane whose byte
// offset falls outside that range is dropped by the hardware's range check,
// so a masked store is still one issued instruction (which keeps hand-counted
// vmcnt waits exact). Word 3 is the gfx9 value (32-bit data format, required
// for untyped access).
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
