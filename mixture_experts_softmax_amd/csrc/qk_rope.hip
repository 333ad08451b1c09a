// QK-Norm + RoPE in one in-place pass, as the NVIDIA Sarvam blog fuses the
// two steps before attention (Table 1, row "QK Norm + RoPE"; the paragraph
// on fused positional embedding): each query and key head is read once,
// RMS-normalised with its learned weight, rotated by its token's position
// and written back.
//
// One workgroup per token, one lane per 16 bytes of its query and key heads
// (LPH lanes per head, all in one wave). Each lane issues its loads first;
// while they are in flight the first HD/2 lanes evaluate the token's rotation
// table into LDS, one pair each (angle p * theta^(-2i/HD) in float64). After
// the barrier the head's sum of squares is reduced across its lanes by xor
// shuffles, and each lane normalises, rotates (the partner half comes from
// lane ^ LPH/2 for the halves pairing; interleaved pairs lie within the lane)
// and stores. One table per token: a table per wave costs more in fp64
// arithmetic than the barrier it saves.
// HBM-bound: every byte of the q and k heads is read once and written once.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "moe.h"

namespace moe {
namespace {

template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16
  static constexpr int kVec = 8;
  __device__ static float load(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t store(float v) { return f32_to_bf16(v); }
};
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load(float v) { return v; }
  __device__ static float store(float v) { return v; }
};

// cos/sin of pair i at position pos: the frequency theta^(-2i/HD) and the
// angle in float64, reduced to [-pi, pi] in float64, then float32 sincos of
// the reduced angle (absolute error ~1e-7 for any int32 position).
template <int HD>
__device__ inline float2 rope_cs(int i, int pos, double log2_theta) {
  const double inv = exp2(-2.0 * i / HD * log2_theta);
  const double ang = (double)pos * inv;
  const double r = ang - rint(ang * 0.15915494309189535) * 6.283185307179586;
  float sn, cn;
  sincosf((float)r, &sn, &cn);
  return make_float2(cn, sn);
}

template <typename E, int HD, int STYLE>
__global__ __launch_bounds__(1024) void qk_norm_rope_kernel(E* __restrict__ qkv,
                                                            const int32_t* __restrict__ positions,
                                                            const E* __restrict__ qw,
                                                            const E* __restrict__ kw, int n_q,
                                                            int n_kv, int64_t row_stride,
                                                            int64_t q_off, int64_t k_off,
                                                            float eps, float theta) {
  constexpr int VEC = Elem<E>::kVec;  // elements per 16-byte lane chunk
  constexpr int LPH = HD / VEC;       // lanes per head (divides the wave)
  static_assert(LPH <= kWave && kWave % LPH == 0, "a head must sit in one wave");
  __shared__ float2 cs[HD / 2];       // (cos, sin) of pair i

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = (n_q + n_kv) * LPH;
  E* row = qkv + (size_t)t * row_stride;
  auto chunk_ptr = [&](int ch, const E*& w) {
    const int h = ch / LPH, l = ch % LPH;
    const bool is_q = h < n_q;
    w = (is_q ? qw : kw) + l * VEC;
    return row + (is_q ? q_off + (int64_t)h * HD : k_off + (int64_t)(h - n_q) * HD) + l * VEC;
  };
  // each thread's first chunk is loaded before the table is computed, so
  // the loads' latency overlaps that work
  v4i xr, wr;
  if (tid < nch) {
    const E* w;
    const E* p = chunk_ptr(tid, w);
    xr = *reinterpret_cast<const v4i*>(p);
    wr = *reinterpret_cast<const v4i*>(w);
  }
  if (tid < HD / 2) cs[tid] = rope_cs<HD>(tid, positions[t], log2((double)theta));
  __syncthreads();

  const float inv_hd = 1.0f / HD;
  // blockDim is a multiple of LPH, so a head's lanes run every iteration together
  for (int ch = tid; ch < nch; ch += blockDim.x) {
    const int l = ch % LPH;
    const E* w;
    E* p = chunk_ptr(ch, w);
    E xv[VEC], wv[VEC];
    if (ch == tid) {
      *reinterpret_cast<v4i*>(xv) = xr;
      *reinterpret_cast<v4i*>(wv) = wr;
    } else {
      *reinterpret_cast<v4i*>(xv) = *reinterpret_cast<const v4i*>(p);
      *reinterpret_cast<v4i*>(wv) = *reinterpret_cast<const v4i*>(w);
    }
    float v[VEC];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      v[e] = Elem<E>::load(xv[e]);
      ss = fmaf(v[e], v[e], ss);
    }
#pragma unroll
    for (int m = LPH / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float r = 1.0f / sqrtf(ss * inv_hd + eps);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = v[e] * r * Elem<E>::load(wv[e]);

    float o[VEC];
    if constexpr (STYLE == MOE_ROPE_INTERLEAVED) {
#pragma unroll
      for (int m = 0; m < VEC / 2; ++m) {
        const float2 f = cs[(l * VEC) / 2 + m];
        const float a = v[2 * m], b = v[2 * m + 1];
        o[2 * m] = a * f.x - b * f.y;
        o[2 * m + 1] = a * f.y + b * f.x;
      }
    } else {
      const bool first = l < LPH / 2;
      const int i0 = (first ? l : l - LPH / 2) * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float q = __shfl_xor(v[e], LPH / 2);
        const float2 f = cs[i0 + e];
        // first half: a = own, b = partner; second half: a = partner, b = own
        o[e] = first ? v[e] * f.x - q * f.y : q * f.y + v[e] * f.x;
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) xv[e] = Elem<E>::store(o[e]);
    *reinterpret_cast<v4i*>(p) = *reinterpret_cast<const v4i*>(xv);
  }
}

template <typename E, int HD>
hipError_t launch_hd(const moe_qk_shape_t& s, void* qkv, const int32_t* pos, const void* qw,
                     const void* kw, hipStream_t st) {
  constexpr int LPH = HD / Elem<E>::kVec;
  const int nch = (s.n_q + s.n_kv) * LPH;
  const auto* q = static_cast<const E*>(qw);
  const auto* k = static_cast<const E*>(kw);
  // one thread per 16-byte chunk of the token's heads (looping beyond 1024
  // threads), and at least one per rotation pair for the table, in whole waves
  const int need = std::max(std::min(nch, 1024), HD / 2);
  const int nth = ((need + kWave - 1) / kWave) * kWave;
  if (s.style == MOE_ROPE_INTERLEAVED)
    hipLaunchKernelGGL((qk_norm_rope_kernel<E, HD, MOE_ROPE_INTERLEAVED>), dim3(s.T), dim3(nth), 0,
                       st, static_cast<E*>(qkv), pos, q, k, s.n_q, s.n_kv, s.row_stride,
                       s.q_offset, s.k_offset, s.eps, s.theta);
  else
    hipLaunchKernelGGL((qk_norm_rope_kernel<E, HD, MOE_ROPE_HALVES>), dim3(s.T), dim3(nth), 0, st,
                       static_cast<E*>(qkv), pos, q, k, s.n_q, s.n_kv, s.row_stride, s.q_offset,
                       s.k_offset, s.eps, s.theta);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const moe_qk_shape_t& s, void* qkv, const int32_t* pos, const void* qw,
                    const void* kw, hipStream_t st) {
  switch (s.head_dim) {
    case 64: return launch_hd<E, 64>(s, qkv, pos, qw, kw, st);
    case 128: return launch_hd<E, 128>(s, qkv, pos, qw, kw, st);
    case 256: return launch_hd<E, 256>(s, qkv, pos, qw, kw, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const moe_qk_shape_t& s, void* qkv, const int32_t* positions,
                               const void* q_weight, const void* k_weight, hipStream_t st) {
  if (s.dtype == MOE_DTYPE_BF16)
    return launch_e<uint16_t>(s, qkv, positions, q_weight, k_weight, st);
  return launch_e<float>(s, qkv, positions, q_weight, k_weight, st);
}

}  // namespace moe
