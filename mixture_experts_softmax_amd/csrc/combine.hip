// Gate-weighted combine of the k routed expert outputs of each token plus the
// shared expert's output, y[t] = sum_j w[t, j] * expert_out[pair_to_row[t*k + j]]
// + shared_out[t], summed in that order in float32, one writer per output
// element (no atomics). The InferX page (section 3.3) fuses this scatter/
// gather step with the router's {indices, weights} output.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kCombThreads = 256;
constexpr int kVec = 8;  // bf16 per thread per step (16 bytes)

// One workgroup per token; thread handles 8 consecutive columns per step.
__global__ __launch_bounds__(kCombThreads) void combine_bf16_kernel(
    const uint16_t* __restrict__ eo, const int32_t* __restrict__ p2r, const float* __restrict__ w,
    const uint16_t* __restrict__ so, uint16_t* __restrict__ y, int T, int d, int k) {
  const int t = blockIdx.x;
  const int rows = T * k;
  __shared__ int row_s[MOE_MAX_K];
  __shared__ float w_s[MOE_MAX_K];
  if (threadIdx.x < k) {
    row_s[threadIdx.x] = p2r[(size_t)t * k + threadIdx.x];
    w_s[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * kVec; c < d; c += kCombThreads * kVec) {
    float acc[kVec];
#pragma unroll
    for (int q = 0; q < kVec; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = row_s[j];
      if (r < 0 || r >= rows) continue;
      const float wj = w_s[j];
      const uint4 p = *reinterpret_cast<const uint4*>(eo + (size_t)r * d + c);
      const uint32_t u[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj, bf16_to_f32((uint16_t)(u[q] & 0xffff)), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, bf16_to_f32((uint16_t)(u[q] >> 16)), acc[2 * q + 1]);
      }
    }
    if (so != nullptr) {
      const uint4 p = *reinterpret_cast<const uint4*>(so + (size_t)t * d + c);
      const uint32_t u[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32((uint16_t)(u[q] & 0xffff));
        acc[2 * q + 1] += bf16_to_f32((uint16_t)(u[q] >> 16));
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
    *reinterpret_cast<uint4*>(y + (size_t)t * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(kCombThreads) void combine_f32_kernel(
    const float* __restrict__ eo, const int32_t* __restrict__ p2r, const float* __restrict__ w,
    const float* __restrict__ so, float* __restrict__ y, int T, int d, int k) {
  const int t = blockIdx.x;
  const int rows = T * k;
  for (int c = threadIdx.x; c < d; c += kCombThreads) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = p2r[(size_t)t * k + j];
      if (r < 0 || r >= rows) continue;
      acc = fmaf(w[(size_t)t * k + j], eo[(size_t)r * d + c], acc);
    }
    if (so != nullptr) acc += so[(size_t)t * d + c];
    y[(size_t)t * d + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine_bf16(const uint16_t* expert_out, const int32_t* pair_to_row,
                               const float* w, const uint16_t* shared_out, uint16_t* y, int T,
                               int d, int k, hipStream_t s) {
  hipLaunchKernelGGL(combine_bf16_kernel, dim3(T), dim3(kCombThreads), 0, s, expert_out,
                     pair_to_row, w, shared_out, y, T, d, k);
  return hipGetLastError();
}

hipError_t launch_combine_f32(const float* expert_out, const int32_t* pair_to_row,
                              const float* w, const float* shared_out, float* y, int T, int d,
                              int k, hipStream_t s) {
  hipLaunchKernelGGL(combine_f32_kernel, dim3(T), dim3(kCombThreads), 0, s, expert_out,
                     pair_to_row, w, shared_out, y, T, d, k);
  return hipGetLastError();
}

}  // namespace moe
