// Router: logits GEMM, then softmax + top-k selection with renormalised gate
// weights, and (bf16/FP8 path) per-token FP8 quantisation of x. The NVIDIA
// Sarvam blog (Table 1 row "Router logits and TopK", MoE-routing paragraph)
// fuses logit computation and selection into one kernel to cut launches and
// memory round trips. Here the logits GEMM is split over K so that a decode
// step's few tokens still spread their 4096-deep dot products over enough
// workgroups to have the router weights in flight at once; the selection
// kernel sums the K slices in a fixed order. For a batch of at most 64
// tokens the selection workgroup also performs the whole permutation
// (offsets, rows, FFN work lists), so routing and permutation take two
// launches in all.
//
// Selection rule: the k largest logits, largest first, equal logits ordered
// by lower expert index. Gate weights are the softmax over all E logits
// renormalised over the chosen k, which equals the softmax over the k chosen
// logits alone (the common denominator cancels); the kernel computes the
// latter.
#include <float.h>

#include "common.h"
#include "internal.h"
#include "quant.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int kLogitWaves = 4;
constexpr int kLogitExperts = kLogitWaves * 32;  // experts per logits tile (32 per wave)
constexpr int kLogitChunk = 128;                  // K per pipeline stage (4 MFMA steps)
constexpr int kLogitMinSlice = 256;               // smallest K slice
constexpr int kLogitTargetWgs = 256;              // aim: at least one workgroup per CU
constexpr int kTallTokens = 64;                   // tokens per tall-batch logits workgroup
constexpr int kTallMin = 64;                      // batches above this use the tall kernel
constexpr int kTallMaxChunks = 8;                 // K chunks per slice of the unrolled tall kernel
constexpr int kTopkWaves = 16;      // fused permutation: one 64-token tile per workgroup
constexpr int kTopkWavesTall = 4;   // otherwise 16 tokens per workgroup
constexpr int kTokPerWave = 4;      // 16 lanes per token
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// Logits, bf16, split over K: workgroup (token tile, expert tile, K slice)
// computes 16 tokens x 128 experts over its slice, wave w the experts
// [32 w, 32 w + 32) with bf16 16x16x32 MFMAs, two 128-deep K chunks in flight
// per wave; it writes the raw partial sums (no bias) to part[slice][T][E].
// Blocks past the logits grid quantise x: one token row per wave.
// ---------------------------------------------------------------------------
struct LogitGrid {
  int n_tt, n_et, ks, cps;  // token tiles, expert tiles, K slices, chunks per slice
  int ksplit;               // decode kernel: waves of a workgroup on 4 K slices (1) or on 4
                            // expert groups (0); with 1 it writes ks / 4 partial slices
  int n_logit;              // logits work items
  int n_lblocks;            // logits blocks: n_logit rounded up to a multiple of the XCDs
  int n_quant;              // quantisation workgroups
};

LogitGrid logit_grid(int T, int d, int E, bool quant) {
  LogitGrid g;
  g.n_tt = ceil_div(T, T > kTallMin ? kTallTokens : kRouteTokens);
  g.n_et = ceil_div(E, kLogitExperts);
  const int nch = d / kLogitChunk;
  const int tiles = max(1, g.n_tt * g.n_et);  // T = 0 still sizes one tile
  const int ks_want = ceil_div(kLogitTargetWgs, tiles);
  int ks = max(1, min(ks_want, d / kLogitMinSlice));
  g.cps = ceil_div(nch, ks);
  if (T > kTallMin) {
    // the unrolled tall kernel: the largest of 8, 4, 2 chunks per slice that
    // still gives at least ks_want slices, when it divides the K chunks
    int cps = kTallMaxChunks;
    while (cps > 2 && nch / cps < ks_want) cps /= 2;
    if (nch % cps == 0) g.cps = cps;
  }
  g.ks = ceil_div(nch, g.cps);  // no empty slice
  g.ksplit = (T <= kTallMin && g.ks % kLogitWaves == 0) ? 1 : 0;
  // with ksplit a workgroup takes one 32-expert group over kLogitWaves slices
  g.n_logit = g.ksplit ? g.n_tt * ceil_div(E, 32) * (g.ks / kLogitWaves) : tiles * g.ks;
  g.n_lblocks = (int)align_up(g.n_logit, kXcds);
  g.n_quant = quant ? ceil_div(T, kLogitWaves) : 0;
  return g;
}

__device__ inline void load_chunk(const uint16_t* xr, const uint16_t* w0, const uint16_t* w1,
                                  int k0, v8bf* xa, v8bf* b0, v8bf* b1) {
#pragma unroll
  for (int s = 0; s < kLogitChunk / 32; ++s) {
    xa[s] = *reinterpret_cast<const v8bf*>(xr + k0 + 32 * s);
    b0[s] = *reinterpret_cast<const v8bf*>(w0 + k0 + 32 * s);
    b1[s] = *reinterpret_cast<const v8bf*>(w1 + k0 + 32 * s);
  }
}

// KSPLIT: the four waves take four consecutive K slices of one 32-expert
// group and add their sums through LDS in wave order, so the workgroup
// writes one partial of ks / 4 (the top-k kernel then reads a quarter of the
// partial logits).
template <bool KSPLIT>
__global__ __launch_bounds__(kLogitWaves * kWave) void route_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    LogitGrid g, float* __restrict__ part, uint8_t* __restrict__ xq, float* __restrict__ xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int b = blockIdx.x;
  if (b >= g.n_lblocks) {  // ---- FP8 quantisation of x: s = amax / 448, codes E4M3(x / s) ----
    const int t = (b - g.n_lblocks) * kLogitWaves + wave;
    if (t < T) quantize_row(x + (size_t)t * d, d, lane, xq + (size_t)t * d, xs + t);
    return;
  }
  // blocks are dealt to the XCDs in turn: remap so that one XCD takes a run
  // of consecutive items, which share a K slice of the router weights (a
  // bijection of [0, n_lblocks); items past n_logit have no work)
  const int per_xcd = g.n_lblocks / kXcds;
  const int wi = (b % kXcds) * per_xcd + b / kXcds;
  if (wi >= g.n_logit) return;
  const int tt = wi % g.n_tt;
  int kz, eb, kzo;  // the wave's K slice, its first expert, the output slice
  if constexpr (KSPLIT) {
    const int n_eg = ceil_div(E, 32);
    const int eg = (wi / g.n_tt) % n_eg;
    kzo = wi / (g.n_tt * n_eg);
    kz = kzo * kLogitWaves + wave;
    eb = eg * 32;
  } else {
    const int et = (wi / g.n_tt) % g.n_et;
    kz = wi / (g.n_tt * g.n_et);
    kzo = kz;
    eb = et * kLogitExperts + wave * 32;
  }

  const int tok = min(tt * kRouteTokens + (lane & 15), T - 1);
  const int kq = (lane >> 4) * 8;  // the lane's 8 K elements of each 32-deep MFMA step
  const uint16_t* xr = x + (size_t)tok * d + kq;
  const uint16_t* w0 = wr + (size_t)min(eb + (lane & 15), E - 1) * d + kq;
  const uint16_t* w1 = wr + (size_t)min(eb + 16 + (lane & 15), E - 1) * d + kq;
  const int c0 = kz * g.cps;
  const int c1 = min(c0 + g.cps, d / kLogitChunk);

  constexpr int NS = kLogitChunk / 32;
  v8bf xa[2][NS], b0[2][NS], b1[2][NS];
  v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  // two chunks in flight; every load is issued (tail chunks re-load the last
  // one) so the wait counts stay exact
  load_chunk(xr, w0, w1, c0 * kLogitChunk, xa[0], b0[0], b1[0]);
  load_chunk(xr, w0, w1, min(c0 + 1, c1 - 1) * kLogitChunk, xa[1], b0[1], b1[1]);
  for (int c = c0; c < c1; c += 2) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      a0 = mfma_bf16_16x16x32(xa[0][s], b0[0][s], a0);
      a1 = mfma_bf16_16x16x32(xa[0][s], b1[0][s], a1);
    }
    load_chunk(xr, w0, w1, min(c + 2, c1 - 1) * kLogitChunk, xa[0], b0[0], b1[0]);
    if (c + 1 < c1) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        a0 = mfma_bf16_16x16x32(xa[1][s], b0[1][s], a0);
        a1 = mfma_bf16_16x16x32(xa[1][s], b1[1][s], a1);
      }
    }
    load_chunk(xr, w0, w1, min(c + 3, c1 - 1) * kLogitChunk, xa[1], b0[1], b1[1]);
  }
  if constexpr (KSPLIT) {
    __shared__ v4f red[kLogitWaves][2][kWave];
    red[wave][0][lane] = a0;
    red[wave][1][lane] = a1;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < kLogitWaves; ++w) {
      a0 += red[w][0][lane];
      a1 += red[w][1][lane];
    }
  }
  float* out = part + (size_t)kzo * T * E;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = tt * kRouteTokens + 4 * (lane >> 4) + q;
    const int e = eb + (lane & 15);
    if (t < T) {
      if (e < E) out[(size_t)t * E + e] = a0[q];
      if (e + 16 < E) out[(size_t)t * E + e + 16] = a1[q];
    }
  }
}

// ---------------------------------------------------------------------------
// Logits for tall batches (T > 64): workgroup (64-token tile, 128-expert tile,
// K slice), wave w the tokens [16 w, 16 w + 16) of the tile over all 128
// experts (8 MFMA column blocks, so each x fragment feeds 8 MFMAs). Each
// 128-deep K chunk of the router weights (128 experts x 256 bytes) is staged
// once per workgroup into a double-buffered LDS tile shared by the 4 waves
// (16-byte chunks XOR-swizzled by row, so the 16 rows a fragment read touches
// fall in distinct banks); x fragments come straight from global memory, two
// chunks ahead. Versus the decode kernel's 16-token tiles this reads x once
// instead of once per wave and the weights once per 64 tokens instead of
// once per 16.
// ---------------------------------------------------------------------------
__device__ inline int tall_swz(int r, int q) {  // element offset of 16-byte chunk q of row r
  return r * kLogitChunk + ((q ^ (r & 15)) << 3);
}

//
// CPS > 0: every slice is exactly CPS chunks and the K loop is unrolled, so
// the wait for each chunk's operands counts exactly the loads issued after
// them (a loop with a run-time trip count and a conditional second half
// makes the compiler drain every load in flight once per chunk, prefetches
// included). CPS = 0: any slice length.
template <int CPS>
__global__ __launch_bounds__(kLogitWaves * kWave) void route_logits_tall_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    LogitGrid g, float* __restrict__ part, uint8_t* __restrict__ xq, float* __restrict__ xs) {
  constexpr int NS = kLogitChunk / 32;                        // MFMA K steps per chunk
  constexpr int NB = kLogitExperts / 16;                      // column blocks per wave
  constexpr int WPT = kLogitExperts * kLogitChunk / 8 / (kLogitWaves * kWave);  // 16 B pieces/thread
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][kLogitExperts * kLogitChunk];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int b = blockIdx.x;
  if (b >= g.n_lblocks) {  // ---- FP8 quantisation of x (as in the decode kernel) ----
    const int t = (b - g.n_lblocks) * kLogitWaves + wave;
    if (t < T) quantize_row(x + (size_t)t * d, d, lane, xq + (size_t)t * d, xs + t);
    return;
  }
  const int per_xcd = g.n_lblocks / kXcds;
  const int wi = (b % kXcds) * per_xcd + b / kXcds;
  if (wi >= g.n_logit) return;
  const int tt = wi % g.n_tt;
  const int et = (wi / g.n_tt) % g.n_et;
  const int kz = wi / (g.n_tt * g.n_et);
  const int c0 = kz * g.cps;
  const int c1 = min(c0 + g.cps, d / kLogitChunk);
  const int eb = et * kLogitExperts;

  const int tok = min(tt * kTallTokens + wave * 16 + (lane & 15), T - 1);
  const uint16_t* xr = x + (size_t)tok * d + (lane >> 4) * 8;
  // this thread's pieces of a weight chunk: piece p = tid + 256 i is expert
  // row p / 16, 16-byte column p % 16
  const uint16_t* wsrc[WPT];
  int wdst[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int p = tid + i * kLogitWaves * kWave;
    const int r = p / 16, q = p % 16;
    wsrc[i] = wr + (size_t)min(eb + r, E - 1) * d + q * 8;
    wdst[i] = tall_swz(r, q);
  }
  auto load_x = [&](int c, v8bf (&xa)[NS]) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
      xa[s2] = *reinterpret_cast<const v8bf*>(xr + (size_t)c * kLogitChunk + 32 * s2);
  };
  auto load_w = [&](int c, v4i (&ws)[WPT]) {
#pragma unroll
    for (int i = 0; i < WPT; ++i)
      ws[i] = *reinterpret_cast<const v4i*>(wsrc[i] + (size_t)c * kLogitChunk);
  };
  auto store_w = [&](const v4i (&ws)[WPT], uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) *reinterpret_cast<v4i*>(dst + wdst[i]) = ws[i];
  };

  v8bf xa[2][NS];
  v4i wst[WPT];
  v4f acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  // every load is issued (tail chunks re-load the last one), so the wait
  // counts stay exact
  load_w(c0, wst);
  load_x(c0, xa[0]);
  load_x(min(c0 + 1, c1 - 1), xa[1]);
  store_w(wst, wl[0]);
  load_w(min(c0 + 1, c1 - 1), wst);
  __syncthreads();
  if constexpr (CPS > 0) {
    // chunk i: its 8 weight fragments of each MFMA step are read before the
    // step's MFMAs; the next chunk's weights go to the other LDS stage, and
    // chunk i + 2's weights and x are loaded (none past the slice)
#pragma unroll
    for (int i = 0; i < CPS; ++i) {
      const int h = i & 1;
      const uint16_t* wb = wl[h];
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        v8bf bf[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int r = n * 16 + (lane & 15);
          bf[n] = *reinterpret_cast<const v8bf*>(wb + tall_swz(r, 4 * s2 + (lane >> 4)));
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = mfma_bf16_16x16x32(xa[h][s2], bf[n], acc[n]);
      }
      if (i + 1 < CPS) {
        // the other stage's readers finished at the barrier ending chunk i-1
        store_w(wst, wl[h ^ 1]);
        if (i + 2 < CPS) {
          load_w(c0 + i + 2, wst);
          load_x(c0 + i + 2, xa[h]);
        }
        __syncthreads();
      }
    }
  } else {
  for (int c = c0; c < c1; c += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = c + h;
      if (cc < c1) {
        const uint16_t* wb = wl[h];
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int r = n * 16 + (lane & 15);
            const v8bf bf = *reinterpret_cast<const v8bf*>(wb + tall_swz(r, 4 * s2 + (lane >> 4)));
            acc[n] = mfma_bf16_16x16x32(xa[h][s2], bf, acc[n]);
          }
        }
        // the other buffer's readers finished at the barrier ending chunk cc-1
        store_w(wst, wl[h ^ 1]);
        load_w(min(cc + 2, c1 - 1), wst);
        load_x(min(cc + 2, c1 - 1), xa[h]);
        __syncthreads();
      }
    }
  }
  }
  float* out = part + (size_t)kz * T * E;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int e = eb + n * 16 + (lane & 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = tt * kTallTokens + wave * 16 + 4 * (lane >> 4) + q;
      if (t < T && e < E) out[(size_t)t * E + e] = acc[n][q];
    }
  }
}

// Logits, float32: one wave per token, lane computes experts lane + 64c with a
// sequential float32 dot product (no bias; one K slice).
__global__ __launch_bounds__(kLogitWaves * kWave) void route_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, int T, int d, int E,
    float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kLogitWaves + threadIdx.x / kWave;
  if (t >= T) return;
  const float* xr = x + (size_t)t * d;
  for (int e = lane; e < E; e += kWave) {
    const float* w = wr + (size_t)e * d;
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(xr[i], w[i], acc);
    logits[(size_t)t * E + e] = acc;
  }
}

// ---------------------------------------------------------------------------
// Top-k over the logits of 64 tokens (NW = 16 waves, the fused permutation)
// or 16 (NW = 4 waves, a quarter of a permutation tile: four times the
// workgroups, so a large batch's selection spreads over more CUs). Each wave serves 4 tokens at once: the 16 lanes
// [16q, 16q + 16) take token 4w + q, lane s holding the
// PL = ceil(E/16) experts [s PL, s PL + PL). A logit is the sum of its K
// slices in slice order, plus the bias. k rounds of a 16-lane (value desc,
// index asc) argmax butterfly. Records, per expert, the mask of its tokens
// routed to it; then either writes them into the 64-bit tile masks (the
// permutation's per-tile histogram: its own bits, the scan counts by
// popcount) or, with FUSED (the batch is this one tile), performs the
// permutation itself.
// ---------------------------------------------------------------------------
constexpr int kPerLane16 = MOE_MAX_E / 16;  // logits held per lane, at most

struct TopkPermute {  // FUSED outputs
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_to_row;
  TileHeader* hdr;  // nullptr: no tile lists
  TileEntry* up;
  TileEntry* dn;
  int cap_up, cap_dn, bm;
};

// 16-lane butterfly by DPP (within each row of 16 lanes): lane l exchanges
// with l^1, l^2, then the mirror in its half row and in its row. Every lane
// of a row ends with the same result for any commutative operation.
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

__device__ inline float sum16(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

// 64-bit selection key of (logit v, expert e): float bits mapped so that
// unsigned order is float order, above the complemented index. -0 is taken
// as +0 (equal logits tie on the index). Key 0 is below every real key.
__device__ inline uint64_t logit_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}
__device__ inline int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ inline float key_logit(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int CTRL>
__device__ inline uint64_t max_step_u64(uint64_t v) {
  const uint64_t o = dpp_u64<CTRL>(v);
  return o > v ? o : v;
}
__device__ inline uint64_t max16_u64(uint64_t v) {
  v = max_step_u64<kDppXor1>(v);
  v = max_step_u64<kDppXor2>(v);
  v = max_step_u64<kDppHalfMirror>(v);
  return max_step_u64<kDppMirror>(v);
}

// PL4 > 0: E = 64 PL4, lane logits read as PL4 16-byte vectors per K slice;
// PL4 = 0: any E, scalar reads. Either way every read of a batch of K slices
// is issued before the first is used, and the slices are added in order.
template <bool FUSED, int PL4, int NW>
__global__ __launch_bounds__(NW * kWave) void route_topk_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wts, uint64_t* __restrict__ masks,
    int32_t* __restrict__ counts, TopkPermute po, FfnCall c) {
  __shared__ unsigned long long mask[MOE_MAX_E];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & 15;
  constexpr int TPW = NW * kTokPerWave;             // tokens per workgroup
  static_assert(TPW == kPermTile || TPW == 16, "a workgroup takes a tile or a 16-bit slice");
  const int tl = wave * kTokPerWave + (lane >> 4);  // token within the workgroup
  const int t = blockIdx.x * TPW + tl;
  const bool track = FUSED || masks != nullptr;
  if (track) {
    for (int e = threadIdx.x; e < E; e += NW * kWave) mask[e] = 0ull;
    __syncthreads();
  }
  const bool live = t < T;
  const int tc = min(t, T - 1);
  const int PL = PL4 > 0 ? 4 * PL4 : ceil_div(E, 16);
  const int ebase = sub * PL;
  // bias first (all reads issued together, clamped index; unused past E)
  float bsv[kPerLane16];
#pragma unroll
  for (int cc = 0; cc < kPerLane16; ++cc)
    bsv[cc] = (bias != nullptr && cc < PL) ? bias[min(ebase + cc, E - 1)] : 0.f;
  float v[kPerLane16];
  if constexpr (PL4 > 0) {
    constexpr int ZB = 16 / PL4;  // K slices per batch (16 vectors in flight)
    v4f acc[PL4];
#pragma unroll
    for (int c4 = 0; c4 < PL4; ++c4) acc[c4] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < ks; z0 += ZB) {
      v4f p[ZB][PL4];
#pragma unroll
      for (int zz = 0; zz < ZB; ++zz) {
        const int z = min(z0 + zz, ks - 1);
#pragma unroll
        for (int c4 = 0; c4 < PL4; ++c4)
          p[zz][c4] = *reinterpret_cast<const v4f*>(part + ((size_t)z * T + tc) * E + ebase + 4 * c4);
      }
#pragma unroll
      for (int zz = 0; zz < ZB; ++zz)
        if (z0 + zz < ks) {
#pragma unroll
          for (int c4 = 0; c4 < PL4; ++c4)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[c4][q] += p[zz][c4][q];
        }
    }
#pragma unroll
    for (int c4 = 0; c4 < PL4; ++c4)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * c4 + q] = acc[c4][q];
  } else {
    constexpr int ZB = 2;
#pragma unroll
    for (int cc = 0; cc < kPerLane16; ++cc) v[cc] = 0.f;
    for (int z0 = 0; z0 < ks; z0 += ZB) {
      float p[ZB][kPerLane16];
#pragma unroll
      for (int zz = 0; zz < ZB; ++zz) {
        const int z = min(z0 + zz, ks - 1);
#pragma unroll
        for (int cc = 0; cc < kPerLane16; ++cc)
          p[zz][cc] = part[((size_t)z * T + tc) * E + min(ebase + cc, E - 1)];
      }
#pragma unroll
      for (int zz = 0; zz < ZB; ++zz)
        if (z0 + zz < ks) {
#pragma unroll
          for (int cc = 0; cc < kPerLane16; ++cc) v[cc] += p[zz][cc];
        }
    }
  }
#pragma unroll
  for (int cc = 0; cc < kPerLane16; ++cc) {
    const int e = ebase + cc;
    if (cc < PL) v[cc] = (e < E) ? v[cc] + bsv[cc] : -INFINITY;
  }
  // Selection on 64-bit keys (order-preserving bits of the logit, then the
  // complement of the expert index): the largest key is the largest logit,
  // lowest index first among equal logits. Branch-free: per round the lane's
  // largest remaining key, the row's largest by DPP butterfly, and the owner
  // clears it.
  // KL key slots can be live: 4 PL4 when E = 64 PL4, else all kPerLane16
  constexpr int KL = PL4 > 0 ? 4 * PL4 : kPerLane16;
  uint64_t key[KL];
#pragma unroll
  for (int cc = 0; cc < KL; ++cc) {
    const int e = ebase + cc;
    key[cc] = (cc < PL && e < E) ? logit_key(v[cc], e) : 0ull;
  }
  int my_e = 0;
  float my_v = -FLT_MAX, top = 0.f;
  for (int j = 0; j < k; ++j) {
    // the lane's largest key by a pairwise tree (depth log2 KLP, not KL - 1;
    // slots past KL hold key 0, below every real key)
    constexpr int KLP = KL <= 4 ? 4 : KL <= 8 ? 8 : 16;
    uint64_t m[KLP];
#pragma unroll
    for (int cc = 0; cc < KLP; ++cc) m[cc] = cc < KL ? key[cc] : 0ull;
#pragma unroll
    for (int w = KLP / 2; w >= 1; w /= 2)
#pragma unroll
      for (int cc = 0; cc < w; ++cc) m[cc] = m[cc + w] > m[cc] ? m[cc + w] : m[cc];
    const uint64_t best = max16_u64(m[0]);
#pragma unroll
    for (int cc = 0; cc < KL; ++cc) key[cc] = key[cc] == best ? 0ull : key[cc];
    const int bi = key_expert(best);
    const float bv = key_logit(best);
    if (j == 0) top = bv;
    if (sub == j) {
      my_e = bi;
      my_v = bv;
    }
  }
  const float ex = (sub < k) ? expf(my_v - top) : 0.f;
  const float den = sum16(ex);
  const bool mine = live && sub < k;
  if (mine) {
    ids[(size_t)t * k + sub] = my_e;
    wts[(size_t)t * k + sub] = ex / den;
    if (track) atomicOr(&mask[my_e], 1ull << tl);
  }
  if (!track) return;
  __syncthreads();
  if constexpr (!FUSED) {
    if constexpr (TPW == kPermTile) {
      for (int e = threadIdx.x; e < E; e += NW * kWave) {
        masks[(size_t)blockIdx.x * E + e] = mask[e];
        counts[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
      }
    } else {
      // this workgroup's 16 tokens are bits [16 part, 16 part + 16) of the
      // tile's masks: bytes 2 part, 2 part + 1 of each (the four workgroups
      // of a tile write disjoint bytes; the scan counts by popcount)
      const int tile = blockIdx.x / (kPermTile / TPW), part = blockIdx.x % (kPermTile / TPW);
      for (int e = threadIdx.x; e < E; e += NW * kWave)
        reinterpret_cast<uint16_t*>(masks + (size_t)tile * E + e)[part] = (uint16_t)mask[e];
    }
  } else {
    // the permutation of this one tile: group sizes are the mask popcounts,
    // offsets their exclusive scan (wave 0, 4 experts per lane), a pair's row
    // its group offset plus the number of earlier tokens in the group. The
    // same wave writes the FFN work lists: the groups' M-tile counts scanned
    // alongside, each lane writing the entries of its own groups (the order
    // and `first` indices of emit_tiles: routed groups, then the shared one)
    __shared__ int offs[MOE_MAX_E + 1];
    if (wave == 0) {
      constexpr int per = MOE_MAX_E / kWave;
      int cnt[per], sum = 0;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int e = lane * per + i;
        cnt[i] = (e < E) ? __popcll(mask[e]) : 0;
        sum += cnt[i];
      }
      int acc = wave_incl_scan_dpp(sum) - sum;
      const int row_start = acc;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int e = lane * per + i;
        if (e < E) {
          offs[e] = acc;
          po.offsets[e] = acc;
        }
        acc += cnt[i];
      }
      if (lane == kWave - 1) {
        offs[E] = acc;
        po.offsets[E] = acc;
      }
      if (po.hdr != nullptr)
        emit_tiles_wave<per>(c, po.bm, E, cnt, row_start, lane, po.hdr, po.up, po.dn, po.cap_up,
                             po.cap_dn);
    }
    __syncthreads();
    if (mine) {
      const unsigned long long below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
      const int p = t * k + sub;
      const int row = offs[my_e] + __popcll(mask[my_e] & below);
      po.sorted_pair[row] = p;
      po.pair_to_row[p] = row;
    }
  }
}

}  // namespace

// Rows of partial logits (K slices x tokens) the workspace holds: a bound on
// ks * T that grows with T, so a workspace sized for a batch serves every
// smaller one. ks <= d/256 gives T * max(1, d/256); ks <= ceil(256 / tiles)
// with T <= 16 * token tiles gives T + 4096 / expert tiles.
size_t route_partial_rows(int T, int d, int E) {
  // K slices x tokens: at most d / kLogitMinSlice slices, and (slices =
  // ceil(target / tiles)) at most T + target x tile height / expert tiles
  // rows; the tall kernel's 64-token tiles give the larger second bound
  const size_t n_et = ceil_div(E, kLogitExperts);
  const size_t a = (size_t)T * max(1, d / kLogitMinSlice);
  const size_t b = (size_t)T + ceil_div(kLogitTargetWgs * kTallTokens, (int)n_et);
  // the tall kernel's power-of-two chunk counts give fewer than twice the
  // wanted slices, or d / (8 x 128) slices where the 8-chunk cap binds
  const size_t c = (size_t)T * max(1, d / (kLogitChunk * kTallMaxChunks));
  const size_t bc = 2 * b > c ? 2 * b : c;
  return a < bc ? a : bc;
}

size_t route_ws_bytes(int T, int d, int E) {
  return align_up(route_partial_rows(T, d, E) * E * sizeof(float), 256);
}

hipError_t launch_route(bool bf16, const void* x, const void* w_router, const float* bias, int T,
                        int d, int E, int k, int32_t* ids, float* w, uint8_t* xq, float* x_scale,
                        void* ws, uint64_t* masks, int32_t* counts, const RoutePermute* fuse,
                        hipStream_t s, hipEvent_t after_logits) {
  float* part = static_cast<float*>(ws);
  int ks = 1;
  if (bf16) {
    const LogitGrid g = logit_grid(T, d, E, xq != nullptr);
    ks = g.ksplit ? g.ks / kLogitWaves : g.ks;  // partial slices the top-k sums
    if ((size_t)ks * T > route_partial_rows(T, d, E)) return hipErrorInvalidValue;
    if (T > kTallMin) {
      const bool exact = g.cps * g.ks == d / kLogitChunk;
#define MOE_TALL(C)                                                                      \
  hipLaunchKernelGGL(route_logits_tall_kernel<C>, dim3(g.n_lblocks + g.n_quant),         \
                     dim3(kLogitWaves * kWave), 0, s, static_cast<const uint16_t*>(x), \
                     static_cast<const uint16_t*>(w_router), T, d, E, g, part, xq, x_scale)
      if (exact && g.cps == 8)
        MOE_TALL(8);
      else if (exact && g.cps == 4)
        MOE_TALL(4);
      else if (exact && g.cps == 2)
        MOE_TALL(2);
      else
        MOE_TALL(0);
#undef MOE_TALL
    } else if (g.ksplit) {
      hipLaunchKernelGGL(route_logits_bf16_kernel<true>, dim3(g.n_lblocks + g.n_quant),
                         dim3(kLogitWaves * kWave), 0, s, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), T, d, E, g, part, xq, x_scale);
    } else {
      hipLaunchKernelGGL(route_logits_bf16_kernel<false>, dim3(g.n_lblocks + g.n_quant),
                         dim3(kLogitWaves * kWave), 0, s, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), T, d, E, g, part, xq, x_scale);
    }
  } else {
    hipLaunchKernelGGL(route_logits_f32_kernel, dim3(ceil_div(T, kLogitWaves)),
                       dim3(kLogitWaves * kWave), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(w_router), T, d, E, part);
  }
  if (after_logits != nullptr) {  // x codes and scales are written: the caller may fork
    const hipError_t e = hipEventRecord(after_logits, s);
    if (e != hipSuccess) return e;
  }
  // fused: one workgroup of 16 waves; otherwise 16-token workgroups, four
  // per 64-token tile (past T too, so every byte of the masks is written)
  const dim3 grid_f(ceil_div(T, kPermTile)), block_f(kTopkWaves * kWave);
  const dim3 grid_t(ceil_div(T, kPermTile) * (kPermTile / (kTopkWavesTall * kTokPerWave))),
      block_t(kTopkWavesTall * kWave);
  TopkPermute po{};
  FfnCall c{};
  if (fuse != nullptr && T <= kPermTile) {
    po.offsets = fuse->offsets;
    po.sorted_pair = fuse->sorted_pair;
    po.pair_to_row = fuse->pair_to_row;
    if (fuse->c != nullptr && fuse->tiles_ws != nullptr) {
      c = *fuse->c;
      po.bm = fuse->bm;
      tile_lists(c, po.bm, fuse->tiles_ws, &po.hdr, &po.up, &po.dn, &po.cap_up, &po.cap_dn);
    }
  }
  const bool fused = po.offsets != nullptr;
  const int pl4 = (E % 64 == 0) ? E / 64 : 0;
#define MOE_TOPK(F, P)                                                                       \
  if constexpr (F)                                                                            \
    hipLaunchKernelGGL((route_topk_kernel<F, P, kTopkWaves>), grid_f, block_f, 0, s, part, ks, \
                       bias, T, E, k, ids, w, masks, counts, po, c);                          \
  else                                                                                        \
    hipLaunchKernelGGL((route_topk_kernel<F, P, kTopkWavesTall>), grid_t, block_t, 0, s, part, \
                       ks, bias, T, E, k, ids, w, masks, counts, po, c)
#define MOE_TOPK_F(F)        \
  switch (pl4) {             \
    case 1: MOE_TOPK(F, 1); break; \
    case 2: MOE_TOPK(F, 2); break; \
    case 3: MOE_TOPK(F, 3); break; \
    case 4: MOE_TOPK(F, 4); break; \
    default: MOE_TOPK(F, 0); break; \
  }
  if (fused) {
    MOE_TOPK_F(true)
  } else {
    MOE_TOPK_F(false)
  }
#undef MOE_TOPK_F
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
