// Permutation of (token, slot) pairs into expert-contiguous rows, ascending
// token order inside each expert's group (the scatter the InferX page, section
// 3.3, places after its top-k router). Deterministic and atomic-free in global
// memory:
//   1. count:   per 64-token tile, a 64-bit token mask per expert in LDS
//               (ds_or), its popcount is the tile's count for that expert;
//   2. scan:    per expert, exclusive prefix over tiles; exclusive prefix over
//               experts of the totals gives offsets[E+1];
//   3. scatter: row = offsets[e] + tile prefix[e] + popcount(mask[e] below the
//               token's lane).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kScanThreads = 256;  // >= MOE_MAX_E

// Builds the per-expert token masks of one 64-token tile in LDS.
__device__ void tile_masks(const int32_t* __restrict__ ids, int T, int E, int k,
                           unsigned long long* mask) {
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kPermTile) mask[e] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kPermTile + lane;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPermTile) void perm_count_kernel(const int32_t* __restrict__ ids,
                                                               int T, int E, int k,
                                                               int32_t* __restrict__ counts) {
  __shared__ unsigned long long mask[256];
  tile_masks(ids, T, E, k, mask);
  for (int e = threadIdx.x; e < E; e += kPermTile)
    counts[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
}

// One workgroup: per-expert scan over tiles (counts -> tile bases in place)
// and the exclusive scan over experts.
__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(int32_t* __restrict__ counts,
                                                                 int ntiles, int E,
                                                                 int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kScanThreads];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int t = 0; t < ntiles; ++t) {
      const int c = counts[(size_t)t * E + e];
      counts[(size_t)t * E + e] = run;
      run += c;
    }
  }
  tot[e] = (e < E) ? run : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over kScanThreads entries
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int v = (e >= o) ? tot[e - o] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = tot[e];
  if (e == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(kPermTile) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int E, int k, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_to_row) {
  __shared__ unsigned long long mask[256];
  tile_masks(ids, T, E, k, mask);
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kPermTile + lane;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = ids[p];
    if (e < 0 || e >= E) {
      pair_to_row[p] = -1;
      continue;
    }
    const int row = offsets[e] + base[(size_t)blockIdx.x * E + e] + __popcll(mask[e] & below);
    sorted_pair[row] = p;
    pair_to_row[p] = row;
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int E) {
  return align_up((size_t)ceil_div(T, kPermTile) * E * sizeof(int32_t), 256);
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_row, void* ws, hipStream_t s) {
  const int ntiles = ceil_div(T, kPermTile);
  int32_t* counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(perm_count_kernel, dim3(ntiles), dim3(kPermTile), 0, s, ids, T, E, k,
                     counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, ntiles, E,
                     offsets);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(ntiles), dim3(kPermTile), 0, s, ids, T, E, k,
                     counts, offsets, sorted_pair, pair_to_row);
  return hipGetLastError();
}

}  // namespace moe
