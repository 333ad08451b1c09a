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
constexpr int kVec = 8;                           // bf16 per thread (16 bytes)
constexpr int kCombCols = kCombThreads * kVec;    // columns per workgroup

__device__ inline void acc8(float* acc, const v4i& p, float wj, bool use) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = bf16_to_f32((uint16_t)((uint32_t)p[q] & 0xffff));
    const float hi = bf16_to_f32((uint16_t)((uint32_t)p[q] >> 16));
    acc[2 * q] = use ? fmaf(wj, lo, acc[2 * q]) : acc[2 * q];
    acc[2 * q + 1] = use ? fmaf(wj, hi, acc[2 * q + 1]) : acc[2 * q + 1];
  }
}

// Workgroup (token, 2048-column chunk); each thread 8 consecutive columns.
// The k expert rows (KMAX >= k slots, slots past k re-read row k-1 and are
// not added) and the shared row are all loaded before the first is summed;
// a pair without a row (pair_to_row outside [0, T k)) adds nothing.
template <int KMAX>
__global__ __launch_bounds__(kCombThreads) void combine_bf16_kernel(
    const uint16_t* __restrict__ eo, const int32_t* __restrict__ p2r, const float* __restrict__ w,
    const uint16_t* __restrict__ so, uint16_t* __restrict__ y, int T, int d, int k) {
  const int chunks = ceil_div(d, kCombCols);
  const int t = blockIdx.x / chunks;
  const int c = (blockIdx.x % chunks) * kCombCols + threadIdx.x * kVec;
  if (c >= d) return;
  const int rows = T * k;
  int r[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = min(j, k - 1);
    r[j] = p2r[(size_t)t * k + jj];
    wj[j] = w[(size_t)t * k + jj];
  }
  v4i p[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int rr = (r[j] >= 0 && r[j] < rows) ? r[j] : 0;
    p[j] = *reinterpret_cast<const v4i*>(eo + (size_t)rr * d + c);
  }
  v4i ps = {0, 0, 0, 0};
  if (so != nullptr) ps = *reinterpret_cast<const v4i*>(so + (size_t)t * d + c);
  float acc[kVec];
#pragma unroll
  for (int q = 0; q < kVec; ++q) acc[q] = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) acc8(acc, p[j], wj[j], j < k && r[j] >= 0 && r[j] < rows);
  if (so != nullptr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_to_f32((uint16_t)((uint32_t)ps[q] & 0xffff));
      acc[2 * q + 1] += bf16_to_f32((uint16_t)((uint32_t)ps[q] >> 16));
    }
  }
  v4i o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (int)((uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16));
  *reinterpret_cast<v4i*>(y + (size_t)t * d + c) = o;
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
  const dim3 grid((unsigned)(T * ceil_div(d, kCombCols))), block(kCombThreads);
#define MOE_COMBINE(KM)                                                                       \
  hipLaunchKernelGGL(combine_bf16_kernel<KM>, grid, block, 0, s, expert_out, pair_to_row, w, \
                     shared_out, y, T, d, k)
  if (k <= 2)
    MOE_COMBINE(2);
  else if (k <= 4)
    MOE_COMBINE(4);
  else if (k <= 8)
    MOE_COMBINE(8);
  else
    MOE_COMBINE(16);
#undef MOE_COMBINE
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
