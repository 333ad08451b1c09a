// Permutation of (token, slot) pairs into expert-contiguous rows, ascending
// token order inside each expert's group (the scatter the InferX page, section
// 3.3, places after its top-k router). Deterministic, no global atomics:
//   1. count:   per 64-token tile, a 64-bit token mask per expert (ds_or in
//               LDS). The layer path gets the masks from the top-k kernel
//               instead (each of its workgroups writes a 16-token slice).
//   2. scan:    one workgroup; per expert an exclusive prefix over tiles (tile
//               counts staged through LDS in chunks), then an exclusive prefix
//               over experts gives offsets[E+1]. In the layer path the same
//               workgroup also writes the grouped-FFN tile lists, since it is
//               the first to know every group's size.
//   3. scatter: row = offsets[e] + tile base[e] + popcount(mask[e] below the
//               token's lane).
//   4. gather (optional, moe_permute only): the FP8 rows of x and their
//               scales copied into grouped-row order. The layer path skips it:
//               its GEMMs read x's rows through sorted_pair while staging them.
#include "common.h"
#include "internal.h"
#include "quant.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanStage = 8192;  // tile counts staged per chunk (32 KiB of LDS)

__global__ __launch_bounds__(kPermTile) void perm_count_kernel(const int32_t* __restrict__ ids,
                                                               int T, int E, int k,
                                                               uint64_t* __restrict__ masks,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ tile_counts) {
  __shared__ unsigned long long mask[MOE_MAX_E];
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
  for (int e = lane; e < E; e += kPermTile) {
    const int n = __popcll(mask[e]);
    masks[(size_t)blockIdx.x * E + e] = mask[e];
    counts[(size_t)blockIdx.x * E + e] = n;
    if (tile_counts != nullptr) tile_counts[(size_t)blockIdx.x * E + e] = n;
  }
}

// Tile counts from tile masks: out[i] = popcount(masks[i]) for i < n.
__global__ __launch_bounds__(256) void perm_popcount_kernel(const uint64_t* __restrict__ masks,
                                                            int n, int32_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = __popcll(masks[i]);
}

// Gather of the FP8 activation rows into grouped-row order: row r < offsets[E]
// gets xq[sorted_pair[r] / k] and its scale. One wave per row, 16-byte pieces,
// every load of a lane issued before its first store.
constexpr int kGatherRows = 4;  // rows (waves) per workgroup
constexpr int kGatherMaxPieces = MOE_MAX_D / 16 / kWave;

__global__ __launch_bounds__(kGatherRows * kWave) void perm_gather_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ sorted_pair, const int32_t* __restrict__ offsets, int E, int k,
    int d, int max_rows, uint8_t* __restrict__ x_perm, float* __restrict__ x_perm_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * kGatherRows + threadIdx.x / kWave;
  if (r >= min(offsets[E], max_rows)) return;
  const int t = sorted_pair[r] / k;
  const int pieces = d / 16;  // d is a multiple of 128: whole pieces
  const v4i* src = reinterpret_cast<const v4i*>(xq + (size_t)t * d);
  v4i* dst = reinterpret_cast<v4i*>(x_perm + (size_t)r * d);
  v4i v[kGatherMaxPieces];
#pragma unroll
  for (int i = 0; i < kGatherMaxPieces; ++i)
    if (lane + i * kWave < pieces) v[i] = src[lane + i * kWave];
#pragma unroll
  for (int i = 0; i < kGatherMaxPieces; ++i)
    if (lane + i * kWave < pieces) dst[lane + i * kWave] = v[i];
  if (lane == 0) x_perm_scale[r] = x_scale[t];
}

// Workgroup 0 scans. Tile counts are the popcounts of the tile masks; counts
// [ntiles][E] receives the per-tile bases. With
// hdr != nullptr also emits the tile lists of `c` (set 0 = the E routed
// groups with these offsets, set 1 = the shared expert if present).
// Workgroups 1, 2, ... (q.T > 0) quantise x to FP8, one token row per wave:
// the scan occupies one CU, so the rows are quantised on the others.
__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(
    const uint64_t* __restrict__ masks, int32_t* __restrict__ counts, int ntiles, int E,
    int32_t* __restrict__ offsets, FfnCall c,
    int bm, TileHeader* hdr, TileEntry* up, TileEntry* down, int cap_up, int cap_dn,
    QuantRows q) {
  __shared__ int stage[kScanStage];
  __shared__ int tot[MOE_MAX_E];
  __shared__ TileLds L;
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const int t = (blockIdx.x - 1) * (kScanThreads / kWave) + tid / kWave;
    if (t < q.T)
      quantize_row(q.x + (size_t)t * q.d, q.d, tid & (kWave - 1), q.xq + (size_t)t * q.d,
                   q.xs + t);
    return;
  }
  int run = 0;
  const int ct = kScanStage / E;  // tiles per chunk
  for (int t0 = 0; t0 < ntiles; t0 += ct) {
    const int nt = min(ct, ntiles - t0);
    for (int i = tid; i < nt * E; i += kScanThreads) stage[i] = __popcll(masks[(size_t)t0 * E + i]);
    __syncthreads();
    if (tid < E) {
      for (int t = 0; t < nt; ++t) {
        const int v = stage[t * E + tid];
        stage[t * E + tid] = run;
        run += v;
      }
    }
    __syncthreads();
    for (int i = tid; i < nt * E; i += kScanThreads) counts[(size_t)t0 * E + i] = stage[i];
    __syncthreads();
  }
  // inclusive scan of the per-expert totals, by wave 0 (4 experts per lane)
  if (tid < E) tot[tid] = run;
  __syncthreads();
  if (tid < kWave) {
    constexpr int per = MOE_MAX_E / kWave;
    int v[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      v[i] = (e < E) ? tot[e] : 0;
      sum += v[i];
    }
    int acc = wave_incl_scan(sum, tid) - sum;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      acc += v[i];
      if (e < E) {
        tot[e] = acc;
        offsets[e + 1] = acc;
      }
    }
    if (tid == 0) offsets[0] = 0;
  }
  __syncthreads();
  if (hdr == nullptr) return;

  // groups: routed experts (set 0), then the shared expert (set 1)
  const int NG = E + (c.nsets > 1 ? 1 : 0);
  for (int i = tid; i < NG; i += kScanThreads) {
    if (i < E) {
      L.g_row0[i] = (i == 0) ? 0 : tot[i - 1];
      L.g_rows[i] = tot[i] - L.g_row0[i];
      L.g_set[i] = 0;
    } else {
      L.g_row0[i] = 0;
      L.g_rows[i] = min(c.set[1].rows_fixed, c.set[1].max_rows);
      L.g_set[i] = 1;
    }
  }
  __syncthreads();
  emit_tiles(c, bm, NG, E, L, hdr, up, down, cap_up, cap_dn);
}

__global__ __launch_bounds__(kPermTile) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int E, int k, const uint64_t* __restrict__ masks,
    const int32_t* __restrict__ bases, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kPermTile + lane;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const size_t tb = (size_t)blockIdx.x * E;
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = ids[p];
    if (e < 0 || e >= E) {
      pair_to_row[p] = -1;
      continue;
    }
    const int row = offsets[e] + bases[tb + e] + __popcll(masks[tb + e] & below);
    sorted_pair[row] = p;
    pair_to_row[p] = row;
  }
}

}  // namespace

size_t perm_masks_bytes(int T, int E) {
  return align_up((size_t)ceil_div(T, kPermTile) * E * sizeof(uint64_t), 256);
}
size_t perm_counts_bytes(int T, int E) {
  return align_up((size_t)ceil_div(T, kPermTile) * E * sizeof(int32_t), 256);
}
size_t permute_ws_bytes(int T, int E) { return perm_masks_bytes(T, E) + perm_counts_bytes(T, E); }

hipError_t launch_perm_scan_scatter(const int32_t* ids, int T, int E, int k, uint64_t* masks,
                                    int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                    int32_t* pair_to_row, const FfnCall* c, int bm, void* tiles_ws,
                                    hipStream_t s, const QuantRows* quant) {
  const int ntiles = ceil_div(T, kPermTile);
  TileHeader* hdr = nullptr;
  TileEntry *up = nullptr, *dn = nullptr;
  int cap_up = 0, cap_dn = 0;
  FfnCall cc{};
  if (c != nullptr && tiles_ws != nullptr) {
    cc = *c;
    tile_lists(cc, bm, tiles_ws, &hdr, &up, &dn, &cap_up, &cap_dn);
  }
  QuantRows q{};
  if (quant != nullptr) q = *quant;
  const int nq = ceil_div(q.T, kScanThreads / kWave);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1 + nq), dim3(kScanThreads), 0, s, masks, counts,
                     ntiles, E, offsets, cc, bm, hdr, up, dn, cap_up, cap_dn, q);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(ntiles), dim3(kPermTile), 0, s, ids, T, E, k, masks,
                     counts, offsets, sorted_pair, pair_to_row);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_row, int32_t* tile_counts,
                          void* ws, hipStream_t s) {
  uint64_t* masks = static_cast<uint64_t*>(ws);
  int32_t* counts =
      reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + perm_masks_bytes(T, E));
  hipLaunchKernelGGL(perm_count_kernel, dim3(ceil_div(T, kPermTile)), dim3(kPermTile), 0, s, ids,
                     T, E, k, masks, counts, tile_counts);
  return launch_perm_scan_scatter(ids, T, E, k, masks, counts, offsets, sorted_pair, pair_to_row,
                                  nullptr, 0, nullptr, s, nullptr);
}

hipError_t launch_tile_counts(const uint64_t* masks, int T, int E, int32_t* tile_counts,
                              hipStream_t s) {
  const int n = ceil_div(T, kPermTile) * E;
  hipLaunchKernelGGL(perm_popcount_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, s, masks, n,
                     tile_counts);
  return hipGetLastError();
}

hipError_t launch_perm_gather(const uint8_t* xq, const float* x_scale, const int32_t* sorted_pair,
                              const int32_t* offsets, int T, int E, int k, int d, uint8_t* x_perm,
                              float* x_perm_scale, hipStream_t s) {
  const int rows = T * k;
  hipLaunchKernelGGL(perm_gather_kernel, dim3(ceil_div(rows, kGatherRows)),
                     dim3(kGatherRows * kWave), 0, s, xq, x_scale, sorted_pair, offsets, E, k, d,
                     rows, x_perm, x_perm_scale);
  return hipGetLastError();
}

}  // namespace moe
