// Router: logits GEMM, then softmax + top-k selection with renormalised gate
// weights, and (bf16/FP8 path) per-token FP8 quantisation of x. The NVIDIA
// Sarvam blog (Table 1 row "Router logits and TopK", MoE-routing paragraph)
// fuses logit computation and selection into one kernel to cut launches and
// memory round trips; here the logits of a token tile never leave the L2
// between the two kernels, and the split buys parallelism: a T=64 decode
// step spreads its 4096-deep dot products over 16 workgroups x 4 waves
// instead of 4 workgroups.
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

constexpr int kLogitWaves = 4;     // K split across the waves of a logits tile
constexpr int kLogitExperts = 32;  // experts per logits tile (2 MFMA column tiles)
constexpr int kTopkWaves = 16;     // one 64-token tile per top-k workgroup
constexpr int kTokPerWave = kPermTile / kTopkWaves;

constexpr int kQuantGroup = 8;  // 16-byte loads per lane in flight per group

__device__ inline float absmax8(const v4i& c, float m) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)c[q] & 0xffff))));
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)c[q] >> 16))));
  }
  return m;
}

__device__ inline uint2 encode8(const v4i& c, float s) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t c0 = e4m3_encode(__fdiv_rn(bf16_to_f32((uint16_t)((uint32_t)c[q] & 0xffff)), s));
    const uint32_t c1 = e4m3_encode(__fdiv_rn(bf16_to_f32((uint16_t)((uint32_t)c[q] >> 16)), s));
    const uint32_t pair = c0 | (c1 << 8);
    if (q < 2)
      lo |= pair << (16 * q);
    else
      hi |= pair << (16 * (q - 2));
  }
  return make_uint2(lo, hi);
}

// One wave quantises one bf16 row of length d (a multiple of 8) to FP8 E4M3
// with scale amax/448: an amax pass and an encode pass, each issuing its
// 16-byte loads in groups of 8 per lane.
__device__ inline void quantize_row(const uint16_t* __restrict__ xr, int d, int lane,
                                    uint8_t* __restrict__ qr, float* __restrict__ s_out) {
  const int nch = d / 8;  // 8-element chunks in the row
  float amax = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kWave * kQuantGroup) {
    v4i v[kQuantGroup];
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = c0 + i * kWave + lane;
      v[i] = (c < nch) ? *reinterpret_cast<const v4i*>(xr + (size_t)c * 8) : v4i{0, 0, 0, 0};
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
      const int c = c0 + i * kWave + lane;
      v[i] = (c < nch) ? *reinterpret_cast<const v4i*>(xr + (size_t)c * 8) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kQuantGroup; ++i) {
      const int c = c0 + i * kWave + lane;
      if (c < nch) *reinterpret_cast<uint2*>(qr + (size_t)c * 8) = encode8(v[i], s);
    }
  }
  if (lane == 0) *s_out = s;
}

// ---------------------------------------------------------------------------
// Logits, bf16: tile = 16 tokens x 32 experts; wave w accumulates K range
// [w*d/4, (w+1)*d/4) with bf16 16x16x32 MFMAs; the partial tiles are summed
// in LDS (fixed order: wave 0..3). The workgroups of a token tile also
// quantise its tokens' x rows to FP8.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kLogitWaves * kWave) void route_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, float* __restrict__ logits,
    uint8_t* __restrict__ xq, float* __restrict__ xs) {
  __shared__ float part[kLogitWaves][kRouteTokens][kLogitExperts + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tok0 = blockIdx.x * kRouteTokens;
  const int e0 = blockIdx.y * kLogitExperts;

  const int tok = min(tok0 + (lane & 15), T - 1);
  const int kslice = d / kLogitWaves;
  const int kbeg = wave * kslice + (lane >> 4) * 8;
  const uint16_t* xrow = x + (size_t)tok * d + kbeg;
  const uint16_t* w0 = wr + (size_t)min(e0 + (lane & 15), E - 1) * d + kbeg;
  const uint16_t* w1 = wr + (size_t)min(e0 + 16 + (lane & 15), E - 1) * d + kbeg;
  v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int k0 = 0; k0 < kslice; k0 += 32) {
    const v8bf xa = *reinterpret_cast<const v8bf*>(xrow + k0);
    const v8bf b0 = *reinterpret_cast<const v8bf*>(w0 + k0);
    const v8bf b1 = *reinterpret_cast<const v8bf*>(w1 + k0);
    a0 = mfma_bf16_16x16x32(xa, b0, a0);
    a1 = mfma_bf16_16x16x32(xa, b1, a1);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    part[wave][4 * (lane >> 4) + q][lane & 15] = a0[q];
    part[wave][4 * (lane >> 4) + q][16 + (lane & 15)] = a1[q];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRouteTokens * kLogitExperts; i += kLogitWaves * kWave) {
    const int r = i / kLogitExperts, c = i % kLogitExperts;
    const int t = tok0 + r, e = e0 + c;
    if (t < T && e < E) {
      float v = part[0][r][c];
#pragma unroll
      for (int w = 1; w < kLogitWaves; ++w) v += part[w][r][c];
      logits[(size_t)t * E + e] = v + (bias != nullptr ? bias[e] : 0.f);
    }
  }

  // ---- FP8 quantisation of x, per token: s = amax / 448, codes E4M3(x / s) ----
  // The tile's 16 tokens are shared out over the gridDim.y workgroups of this
  // token tile and their waves.
  if (xq == nullptr) return;
  const int nq = kLogitWaves * (int)gridDim.y;  // quantising waves per token tile
  for (int r = blockIdx.y * kLogitWaves + wave; r < kRouteTokens; r += nq) {
    const int t = tok0 + r;
    if (t >= T) break;
    quantize_row(x + (size_t)t * d, d, lane, xq + (size_t)t * d, xs + t);
  }
}

// Logits, float32: one wave per token, lane computes experts lane + 64c with a
// sequential float32 dot product.
__global__ __launch_bounds__(kLogitWaves * kWave) void route_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kLogitWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* xr = x + (size_t)t * d;
  for (int e = lane; e < E; e += kWave) {
    const float* w = wr + (size_t)e * d;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(xr[i], w[i], acc);
    logits[(size_t)t * E + e] = acc + (bias != nullptr ? bias[e] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Top-k over the logits of one 64-token tile. Each wave serves 4 tokens at
// once: the 16 lanes [16q, 16q + 16) take token 4w + q, lane holding experts
// (lane % 16) + 16c. k rounds of a 16-lane (value desc, index asc) argmax
// butterfly. Optionally records, per expert, the 64-bit mask of the tile's
// tokens routed to it and its popcount (the permutation's per-tile histogram).
// ---------------------------------------------------------------------------
constexpr int kPerLane16 = MOE_MAX_E / 16;  // logits held per lane

__global__ __launch_bounds__(kTopkWaves * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, uint64_t* __restrict__ masks, int32_t* __restrict__ counts) {
  __shared__ unsigned long long mask[MOE_MAX_E];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & 15;
  const int tl = wave * kTokPerWave + (lane >> 4);  // token within the tile
  const int t = blockIdx.x * kPermTile + tl;
  if (masks != nullptr) {
    for (int e = threadIdx.x; e < E; e += kTopkWaves * kWave) mask[e] = 0ull;
    __syncthreads();
  }
  const bool live = t < T;
  const float* lr = logits + (size_t)min(t, T - 1) * E;
  float v[kPerLane16];
#pragma unroll
  for (int c = 0; c < kPerLane16; ++c) {
    const int e = sub + 16 * c;
    v[c] = (e < E) ? lr[e] : -INFINITY;
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_v = -FLT_MAX, top = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < kPerLane16; ++c) {
      const int e = sub + 16 * c;
      if (e < E && !((taken >> c) & 1u) && (v[c] > bv || (v[c] == bv && e < bi))) {
        bv = v[c];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 15) == sub) taken |= 1u << (bi >> 4);
    if (j == 0) top = bv;
    if (sub == j) {
      my_e = bi;
      my_v = bv;
    }
  }
  const float ex = (sub < k) ? expf(my_v - top) : 0.f;
  float den = ex;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) den += __shfl_xor(den, o, kWave);
  if (live && sub < k) {
    ids[(size_t)t * k + sub] = my_e;
    wts[(size_t)t * k + sub] = ex / den;
    if (masks != nullptr) atomicOr(&mask[my_e], 1ull << tl);
  }
  if (masks != nullptr) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTopkWaves * kWave) {
      masks[(size_t)blockIdx.x * E + e] = mask[e];
      counts[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
    }
  }
}

}  // namespace

size_t route_ws_bytes(int T, int E) { return align_up((size_t)T * E * sizeof(float), 256); }

hipError_t launch_route(bool bf16, const void* x, const void* w_router, const float* bias, int T,
                        int d, int E, int k, int32_t* ids, float* w, uint8_t* xq, float* x_scale,
                        float* logits, uint64_t* masks, int32_t* counts, hipStream_t s) {
  if (bf16) {
    const dim3 grid(ceil_div(T, kRouteTokens), ceil_div(E, kLogitExperts));
    hipLaunchKernelGGL(route_logits_bf16_kernel, grid, dim3(kLogitWaves * kWave), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                       bias, T, d, E, logits, xq, x_scale);
  } else {
    hipLaunchKernelGGL(route_logits_f32_kernel, dim3(ceil_div(T, kLogitWaves)),
                       dim3(kLogitWaves * kWave), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(w_router), bias, T, d, E, logits);
  }
  hipLaunchKernelGGL(route_topk_kernel, dim3(ceil_div(T, kPermTile)), dim3(kTopkWaves * kWave), 0,
                     s, logits, T, E, k, ids, w, masks, counts);
  return hipGetLastError();
}

}  // namespace moe
