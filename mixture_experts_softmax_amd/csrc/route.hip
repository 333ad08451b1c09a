// Router kernels: logits GEMM, softmax + top-k selection with renormalised
// gate weights, and (bf16/FP8 path) per-token FP8 quantisation of x -- one
// kernel per path, as the NVIDIA Sarvam blog's Table 1 row "Router logits and
// TopK" fuses logit computation and selection (its paragraph on MoE routing).
//
// Selection rule: the k largest logits, largest first, equal logits ordered
// by lower expert index. Gate weights are the softmax over all E logits
// renormalised over the chosen k, which equals the softmax over the k chosen
// logits alone (the common denominator cancels); the kernel computes the
// latter.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;
constexpr int kMaxPerLane = 4;  // E <= 256 = 64 lanes * 4
constexpr int kLgStride = 257;  // logits row stride in LDS (E <= 256, +1 pad)

// Wave-cooperative top-k over E <= 256 values held 4 per lane (expert
// lane + 64 * c in slot c; -inf for padding). Writes ids/weights for one token.
__device__ void wave_topk_store(const float (&v)[kMaxPerLane], int E, int k, int lane,
                                int32_t* ids_out, float* w_out) {
  bool taken[kMaxPerLane] = {false, false, false, false};
  int my_e = 0;
  float my_v = -FLT_MAX;
  float top = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < kMaxPerLane; ++c) {
      const int e = lane + kWave * c;
      if (e < E && !taken[c] && (v[c] > bv || (v[c] == bv && e < bi))) {
        bv = v[c];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int c = 0; c < kMaxPerLane; ++c)
        if (bi == lane + kWave * c) taken[c] = true;
    }
    if (j == 0) top = bv;
    if (lane == j) {
      my_e = bi;
      my_v = bv;
    }
  }
  const float ex = (lane < k) ? expf(my_v - top) : 0.f;
  float den = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, kWave);
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / den;
  }
}

// bf16 router: one workgroup per 16 tokens, 4 waves splitting the experts in
// 16-wide MFMA column tiles (bf16 16x16x32, float32 accumulation).
__global__ __launch_bounds__(kRouteWaves * kWave) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, uint8_t* __restrict__ xq, float* __restrict__ xs) {
  __shared__ float lg[kRouteTokens][kLgStride];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tok0 = blockIdx.x * kRouteTokens;
  const int nsub = ceil_div(E, 16);

  // ---- logits: lane holds token row (lane % 16), K slice (lane / 16) * 8 ----
  v4f acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const int tok = min(tok0 + (lane & 15), T - 1);
  const uint16_t* xrow = x + (size_t)tok * d + (lane >> 4) * 8;
  const uint16_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = min((wave + kRouteWaves * i) * 16 + (lane & 15), E - 1);
    wrow[i] = wr + (size_t)e * d + (lane >> 4) * 8;
  }
#pragma unroll 4
  for (int k0 = 0; k0 < d; k0 += 32) {
    const v8bf a = *reinterpret_cast<const v8bf*>(xrow + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (wave + kRouteWaves * i < nsub) {
        const v8bf b = *reinterpret_cast<const v8bf*>(wrow[i] + k0);
        acc[i] = mfma_bf16_16x16x32(a, b, acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = wave + kRouteWaves * i;
    if (s < nsub) {
      const int e = s * 16 + (lane & 15);
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) lg[4 * (lane >> 4) + q][e] = acc[i][q] + b;
    }
  }
  __syncthreads();

  // ---- top-k + gates: wave w handles token rows 4w .. 4w+3 ----
  for (int r = 0; r < 4; ++r) {
    const int row = wave * 4 + r;
    const int t = tok0 + row;
    if (t >= T) break;
    float v[kMaxPerLane];
#pragma unroll
    for (int c = 0; c < kMaxPerLane; ++c) {
      const int e = lane + kWave * c;
      v[c] = (e < E) ? lg[row][e] : -INFINITY;
    }
    wave_topk_store(v, E, k, lane, ids + (size_t)t * k, wts + (size_t)t * k);
  }

  // ---- FP8 quantisation of x, per token: s = amax / 448, codes E4M3(x / s) ----
  for (int r = 0; r < 4; ++r) {
    const int t = tok0 + wave * 4 + r;
    if (t >= T) break;
    const uint16_t* xr = x + (size_t)t * d;
    float amax = 0.f;
    for (int c = lane * 8; c < d; c += kWave * 8) {
      const uint4 p = *reinterpret_cast<const uint4*>(xr + c);
      const uint32_t w4[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(w4[q] & 0xffff))));
        amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(w4[q] >> 16))));
      }
    }
    amax = wave_max(amax);
    const float s = (amax > 0.f) ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
    uint8_t* qr = xq + (size_t)t * d;
    for (int c = lane * 8; c < d; c += kWave * 8) {
      const uint4 p = *reinterpret_cast<const uint4*>(xr + c);
      const uint32_t w4[4] = {p.x, p.y, p.z, p.w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c0 = e4m3_encode(__fdiv_rn(bf16_to_f32((uint16_t)(w4[q] & 0xffff)), s));
        const uint32_t c1 = e4m3_encode(__fdiv_rn(bf16_to_f32((uint16_t)(w4[q] >> 16)), s));
        const uint32_t pair = c0 | (c1 << 8);
        if (q < 2)
          lo |= pair << (16 * q);
        else
          hi |= pair << (16 * (q - 2));
      }
      *reinterpret_cast<uint2*>(qr + c) = make_uint2(lo, hi);
    }
    if (lane == 0) xs[t] = s;
  }
}

// float32 router: one wave per token; lane computes the logits of experts
// lane + 64c with a sequential float32 dot product.
__global__ __launch_bounds__(kRouteWaves * kWave) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* xr = x + (size_t)t * d;
  float v[kMaxPerLane];
#pragma unroll
  for (int c = 0; c < kMaxPerLane; ++c) {
    const int e = lane + kWave * c;
    if (e < E) {
      const float* w = wr + (size_t)e * d;
      float acc = 0.f;
      for (int i = 0; i < d; ++i) acc = fmaf(xr[i], w[i], acc);
      v[c] = acc + (bias != nullptr ? bias[e] : 0.f);
    } else {
      v[c] = -INFINITY;
    }
  }
  wave_topk_store(v, E, k, lane, ids + (size_t)t * k, wts + (size_t)t * k);
}

}  // namespace

hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* w_router, const float* bias,
                             int T, int d, int E, int k, int32_t* ids, float* w, uint8_t* xq,
                             float* x_scale, hipStream_t s) {
  const dim3 grid(ceil_div(T, kRouteTokens)), block(kRouteWaves * kWave);
  hipLaunchKernelGGL(route_bf16_kernel, grid, block, 0, s, x, w_router, bias, T, d, E, k, ids,
                     w, xq, x_scale);
  return hipGetLastError();
}

hipError_t launch_route_f32(const float* x, const float* w_router, const float* bias, int T,
                            int d, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  const dim3 grid(ceil_div(T, kRouteWaves)), block(kRouteWaves * kWave);
  hipLaunchKernelGGL(route_f32_kernel, grid, block, 0, s, x, w_router, bias, T, d, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
