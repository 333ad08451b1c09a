// Grouped SwiGLU expert FFN: the routed experts' grouped GEMMs and the shared
// expert as one more group, as the NVIDIA Sarvam blog runs routed experts as
// grouped GEMM kernels with resident expert weights (section "Performance
// challenges") and the shared expert as a separate computation (Table 1).
//
// FP8 path, per group g, grouped row r with activation row s:
//   gate/up:  gu = (a[s] . w13[g][n]) * a_scale[s] * w13_scale[g][n]   (E4M3 x E4M3 MFMA)
//             h  = silu(gu[n]) * gu[F + n], quantised per (row, 128 columns)
//   down:     out[r][m] = w2_scale[g][m] * sum_b s_h[r][b] * (hq[r][b] . w2[g][m][b])
//
// Work is a device-built list of tiles (group, up to BM rows, one N tile), so
// empty groups cost nothing and the host never reads routing results. Block i
// of a launch takes list entry (i % 8) * ceil(n / 8) + i / 8: consecutive
// entries -- the M tiles of one (group, N tile), then the next N tile of the
// same group -- run on the same XCD (blocks are dealt to the 8 XCDs in turn),
// so a weight tile read by several M tiles, and a group's activation rows, are
// served from that XCD's L2.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"
#include "pipeline.h"
#include "tiles.h"

namespace moe {

namespace {

constexpr int kBK = 128;      // K bytes per MFMA step (FP8 16x16x128)
constexpr int kXcds = 8;
constexpr int kTileThreads = 256;

// Bound on the M-tile entries of one list: per set, its rows in tiles of bm
// plus one partial tile per group.
size_t tiles_cap(const FfnCall& c, int bm) {
  size_t n = 0;
  for (int s = 0; s < c.nsets; ++s) {
    const FfnSet& S = c.set[s];
    n += (size_t)ceil_div(S.max_rows, bm) + (size_t)S.G;
  }
  return n;
}

// ---------------------------------------------------------------------------
// Tile lists from group offsets held in device memory (moe_grouped_ffn).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTileThreads) void ffn_tiles_kernel(FfnCall c, int bm,
                                                                 TileHeader* hdr, TileEntry* up,
                                                                 TileEntry* down, int cap_up,
                                                                 int cap_dn) {
  __shared__ TileLds L;
  const int G0 = c.set[0].G;
  const int NG = G0 + (c.nsets > 1 ? c.set[1].G : 0);
  for (int i = threadIdx.x; i < NG; i += kTileThreads) {
    const int s = (i < G0) ? 0 : 1;
    const int g = (s == 0) ? i : i - G0;
    const FfnSet S = (s == 0) ? c.set[0] : c.set[1];
    // clamp to [0, max_rows] so malformed offsets cannot send a tile outside
    // the buffers (rows of such groups are then simply not computed)
    int r0 = 0, r1 = min(S.rows_fixed, S.max_rows);
    if (S.offsets != nullptr) {
      r0 = min(max(S.offsets[g], 0), S.max_rows);
      r1 = min(max(S.offsets[g + 1], r0), S.max_rows);
    }
    L.g_row0[i] = r0;
    L.g_rows[i] = r1 - r0;
    L.g_set[i] = s;
  }
  __syncthreads();
  emit_tiles(c, bm, NG, G0, L, hdr, up, down, cap_up, cap_dn);
}

// Block -> work tile. The launch covers n_entries x NT items, dealt to the
// XCDs in contiguous runs; item w belongs to list entry w / NT, whose group
// owns items [first NT, (first + mt) NT) in N-tile-major, M-tile-minor order.
// So the blocks of one XCD run the M tiles of one (group, N tile) one after
// the other, sharing that weight tile in the XCD's L2, and a group's tiles
// stay on one XCD. Returns false for blocks with no work.
struct Tile {
  int row0;   // first row, in the set's grouped row space
  int nrows;  // 1..BM
  int gid;    // (set << 16) | group
  int ntile;
};

template <int BM>
__device__ inline bool pick_tile_at(const TileEntry* __restrict__ list, int n_entries, int NT,
                                    int xcd, int slot, Tile& t) {
  const int total = n_entries * NT;
  const int per = ceil_div(total, kXcds);
  const int w = xcd * per + slot;
  if (slot >= per || w >= total) return false;
  const TileEntry te = list[w / NT];
  const int mt = ceil_div(te.rows, BM);
  const int local = w - te.first * NT;
  t.ntile = local / mt;
  const int m = local - t.ntile * mt;
  t.row0 = te.row0 + m * BM;
  t.nrows = min(BM, te.rows - m * BM);
  t.gid = te.gid;
  return true;
}

template <int BM>
__device__ inline bool pick_tile(const TileEntry* __restrict__ list, int n_entries, int NT,
                                 Tile& t) {
  return pick_tile_at<BM>(list, n_entries, NT, blockIdx.x % kXcds, blockIdx.x / kXcds, t);
}

__device__ inline v8i pack8(const v4i& lo, const v4i& hi) {
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Swizzled offset of 16-byte chunk c of row r in a [rows][128 B] LDS tile.
__device__ inline int swz(int r, int c) { return r * kBK + ((c ^ (r & 7)) << 4); }

// A fragment of M subtile i from an LDS tile: row (i*16 + lane%16), bytes
// [(lane/16)*16, +16) and [64 + (lane/16)*16, +16) of the 128-byte K step.
__device__ inline v8i lds_afrag(const uint8_t* tile, int i, int lane) {
  const int r = i * 16 + (lane & 15);
  const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(r, lane >> 4));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(r, 4 + (lane >> 4)));
  return pack8(lo, hi);
}

// B fragment: 16 weight rows, lane reads row (lane%16) at the same byte slices.
__device__ inline v8i glb_bfrag(const uint8_t* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 64);
  return pack8(lo, hi);
}

// MXFP4 weights (OCP Microscaling: E2M1 elements, one E8M0 scale per 32).
// With the A fragment above, lane group j of the FP8 operand holds K
// [16 j, +16) and [64 + 16 j, +16) of the step, which the MFMA pairs with
// K [32 j, +32) of an FP4 operand: 16 packed bytes, low nibble first, one
// contiguous run of one scale block. So a lane reads 16 bytes at packed offset
// 16 j of its row's 64-byte step and the one scale byte of block 4 kt + j,
// which the instruction applies to that lane's 32 elements.
struct Fp4Frag {
  v4i w;
  int s;  // E8M0 scale in the low byte
};

template <bool W4>
using BFrag = typename std::conditional<W4, Fp4Frag, v8i>::type;

// Weight bytes per row and K step (128 K elements).
template <bool W4>
constexpr int kstep_bytes() { return W4 ? kBK / 2 : kBK; }

// Fragment of K step kt. p: the lane's row at its lane-group offset
// ((lane / 16) * 16 bytes); e (MXFP4): the row's scale bytes + lane / 16.
// WS = false (MXFP4): the codes only; the scale comes from the row-resident scales.
template <bool W4, bool WS = true>
__device__ inline BFrag<W4> load_bfrag(const uint8_t* p, const uint8_t* e, int kt) {
  if constexpr (W4)
    return Fp4Frag{*reinterpret_cast<const v4i*>(p + kt * (kBK / 2)), WS ? (int)e[kt * 4] : 0};
  else
    return glb_bfrag(p + kt * kBK);
}

// MXFP4 block scales of a fragment's 16 weight rows over a K loop of KT
// steps, held in registers for the whole loop: a byte load per fragment and
// step costs a cache-line access per row (as many as the codes), and even
// 16-byte loads every four steps re-fetch each row's scale line several times
// from HBM. Instead the 4 lanes of a row (lane groups g = 0..3) each load a
// quarter of the row's 4 KT scale bytes once: lane group g holds the dwords
// of steps [g KT/4, (g + 1) KT/4). Step kt's dword (one byte per lane group)
// is then read from lane (lane % 16) + 16 (kt / (KT/4)) and shifted to the
// lane's byte.
template <int KT>
__device__ inline void load_scale_row(int (&sr)[KT / 4], const uint8_t* row, int lane) {
  const int* p = reinterpret_cast<const int*>(row) + (lane >> 4) * (KT / 4);
#pragma unroll
  for (int t = 0; t < KT / 4; ++t) sr[t] = p[t];
}
template <int KT>
__device__ inline int scale_of_step(const int (&sr)[KT / 4], int kt, int lane) {
  constexpr int DW = KT / 4;
  return __shfl(sr[kt % DW], (lane & 15) + 16 * (kt / DW)) >> (8 * (lane >> 4));
}

// The tall-tile kernels keep their weight rows' scales in LDS instead (the
// registers are taken by the staging): row r's 4 KT scale bytes at dwords
// [r (KT + 1), +KT) -- one dword of padding per row, so the 16 rows of a
// fragment read fall in 16 different banks. Filled once per workgroup by all
// NTH threads, 16 global bytes (4 K steps) per piece; rowp(r) is row r's
// scale bytes in global memory.
template <int KT, int ROWS, int NTH, typename RowPtr>
__device__ inline void fill_scale_tile(int* tile, RowPtr rowp, int tid) {
  constexpr int PPR = KT / 4;  // 16-byte pieces per row
#pragma unroll
  for (int i = 0; i < (ROWS * PPR + NTH - 1) / NTH; ++i) {
    const int p = tid + i * NTH;
    if (ROWS * PPR % NTH == 0 || p < ROWS * PPR) {
      const int r = p / PPR, q = p % PPR;
      const v4i v = *reinterpret_cast<const v4i*>(rowp(r) + 16 * q);
#pragma unroll
      for (int t = 0; t < 4; ++t) tile[r * (KT + 1) + 4 * q + t] = v[t];
    }
  }
}

// The same fill in two halves, so a kernel can issue the loads early and
// write the tile later: a thread's pieces in registers, then into the tile.
template <int KT, int ROWS, int NTH>
constexpr int scale_pieces() { return (ROWS * (KT / 4) + NTH - 1) / NTH; }
template <int KT, int ROWS, int NTH, int NP, typename RowPtr>
__device__ inline void load_scale_pieces(v4i (&v)[NP], RowPtr rowp, int tid) {
  static_assert(NP == scale_pieces<KT, ROWS, NTH>(), "one register per piece");
  constexpr int PPR = KT / 4;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = min(tid + i * NTH, ROWS * PPR - 1);
    v[i] = *reinterpret_cast<const v4i*>(rowp(p / PPR) + 16 * (p % PPR));
  }
}
template <int KT, int ROWS, int NTH, int NP>
__device__ inline void store_scale_pieces(int* tile, const v4i (&v)[NP], int tid) {
  static_assert(NP == scale_pieces<KT, ROWS, NTH>(), "one register per piece");
  constexpr int PPR = KT / 4;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = tid + i * NTH;
    if (ROWS * PPR % NTH == 0 || p < ROWS * PPR) {
      const int r = p / PPR, q = p % PPR;
#pragma unroll
      for (int t = 0; t < 4; ++t) tile[r * (KT + 1) + 4 * q + t] = v[i][t];
    }
  }
}
template <int KT>
__device__ inline int scale_from_tile(const int* tile, int r, int kt, int lane) {
  return reinterpret_cast<const uint8_t*>(tile)[4 * (r * (KT + 1) + kt) + (lane >> 4)];
}


// E4M3 activations x E4M3 weights, or x MXFP4 weights (A scale 2^0, B scale
// per lane from the fragment; the FP4 operand occupies the low 4 registers).
__device__ inline v4f mfma_w(const v8i& a, const v8i& b, const v4f& c) {
  return mfma_fp8_16x16x128(a, b, c);
}
__device__ inline v4f mfma_w(const v8i& a, const Fp4Frag& b, const v4f& c) {
  const v8i bw = v8i{b.w[0], b.w[1], b.w[2], b.w[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 0, 4, 0, 127, 0, b.s);
}
// The same products with the weights as the A operand: lane l then holds the
// four consecutive output channels 4 (l / 16) + q of activation row l % 16.
__device__ inline v4f mfma_wt(const v8i& w, const v8i& x, const v4f& c) {
  return mfma_fp8_16x16x128(w, x, c);
}
__device__ inline v4f mfma_wt(const Fp4Frag& w, const v8i& x, const v4f& c) {
  const v8i ww = v8i{w.w[0], w.w[1], w.w[2], w.w[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ww, x, c, 4, 0, 0, w.s, 0, 127);
}

// The fields of set `sid` (0 or 1), read field by field from the kernel
// arguments so the compiler keeps them in scalar registers.
struct SetView {
  const uint8_t* w13;
  const float* s13;
  const uint8_t* w2;
  const float* s2;
  const uint8_t* e13;
  const uint8_t* e2;
  const int32_t* row_src;
  int src_div, F;
  uint8_t* h;
  float* h_scale;
  void* out;
};

__device__ inline SetView set_view(const FfnCall& c, int sid) {
  SetView v;
  v.w13 = sid ? c.set[1].w13 : c.set[0].w13;
  v.s13 = sid ? c.set[1].s13 : c.set[0].s13;
  v.w2 = sid ? c.set[1].w2 : c.set[0].w2;
  v.s2 = sid ? c.set[1].s2 : c.set[0].s2;
  v.e13 = sid ? c.set[1].e13 : c.set[0].e13;
  v.e2 = sid ? c.set[1].e2 : c.set[0].e2;
  v.row_src = sid ? c.set[1].row_src : c.set[0].row_src;
  v.src_div = sid ? c.set[1].src_div : c.set[0].src_div;
  v.F = sid ? c.set[1].F : c.set[0].F;
  v.h = sid ? c.set[1].h : c.set[0].h;
  v.h_scale = sid ? c.set[1].h_scale : c.set[0].h_scale;
  v.out = sid ? c.set[1].out : c.set[0].out;
  return v;
}

// Activation rows of tile rows r[0..N) (rows past the tile repeat its last
// row; the permutation's entries divided by the set's src_div). The entries
// are loaded under one uniform branch, so the N loads issue back to back: a
// branch per row makes each wait for the one before.
template <int N>
__device__ inline void gather_rows(const Tile& te, const SetView& S, int a_rows, const int (&r)[N],
                                   int (&src)[N]) {
  int grow[N];
#pragma unroll
  for (int i = 0; i < N; ++i) grow[i] = te.row0 + min(r[i], te.nrows - 1);
  if (S.row_src != nullptr) {
#pragma unroll
    for (int i = 0; i < N; ++i) src[i] = S.row_src[grow[i]];
#pragma unroll
    for (int i = 0; i < N; ++i) src[i] /= S.src_div;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) src[i] = grow[i];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) src[i] = min(max(src[i], 0), a_rows - 1);
}

// B operand prefetch depth (K steps of weights in flight per wave), by the
// rows a wave holds (more rows: a bigger accumulator, fewer registers left).
template <int ROWS, int LIMIT>
constexpr int prefetch_depth() { return ROWS <= LIMIT ? 3 : 2; }

// Waves of a GEMM workgroup: 4 along N (each owns a quarter of the tile's
// columns) times WM along M (each owns BM / WM rows). WM = 2 halves every
// wave's accumulator, which buys registers for a deeper weight ring and two
// waves per SIMD; the two M halves read the same weight fragments, the
// second time from the L2.
constexpr int kNWaves = 4;

// The gate/up epilogues' arithmetic, shared so that every gate/up kernel
// writes the same h codes and scales. h = silu(g) u with g, u the scaled
// gate and up values; the row's x scale sx is left out of u (silu(g) u / sx
// is what the epilogues keep) and put back in the block's amax and in the
// code factor: codes = (h / sx) (sx / s), with s = amax |h| / 448.
__device__ inline float silu_times(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}
// s from the block's largest |h / sx| (1 for an all-zero block)
__device__ inline float h_block_scale(float am_over_sx, float sx) {
  const float am = am_over_sx * sx;
  return (am > 0.f) ? __fdiv_rn(am, kE4M3Max) : 1.0f;
}

// Gate/up epilogue, of the register-fed gate/up kernels: x and weight scales,
// SwiGLU, per-(row, 128-column) amax across the kNWaves N waves (through LDS
// `red`), then FP8 h codes and their block scale. acc[i][jj] holds gate
// columns, acc[i][NS + jj] the matching up columns; the wave owns rows
// [rbase, rbase + 16 MS) and h columns [32 wn, 32 wn + 32) of the tile.
template <int BM, int MS, int NS>
__device__ inline void gateup_epilogue(v4f (&acc)[MS][2 * NS], const float* sxl,
                                       float (&red)[kNWaves][BM], const float* sg,
                                       const float* su, int rbase, int wn, int lane,
                                       const Tile& te, const SetView& S, int ntile) {
  constexpr int WN = NS * 16;
  const int F = S.F;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rbase + i * 16 + 4 * (lane >> 4) + q;
      const float sx = sxl[r];
      float m = 0.f;
#pragma unroll
      for (int jj = 0; jj < NS; ++jj) {
        const float gv = acc[i][jj][q] * sx * sg[jj];
        const float hx = silu_times(gv, acc[i][NS + jj][q] * su[jj]);  // h / sx
        acc[i][jj][q] = hx;
        m = fmaxf(m, fabsf(hx));
      }
      m = max16(m);
      if ((lane & 15) == 0) red[wn][r] = m;
    }
  }
  __syncthreads();
  const int hblocks = F / kHN;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rbase + i * 16 + 4 * (lane >> 4) + q;
      if (r >= te.nrows) continue;
      float am = red[0][r];
#pragma unroll
      for (int ww = 1; ww < kNWaves; ++ww) am = fmaxf(am, red[ww][r]);
      const float sx = sxl[r];
      const float s = h_block_scale(am, sx);
      const float f = sx * __builtin_amdgcn_rcpf(s);
      const size_t grow = (size_t)(te.row0 + r);
      uint8_t* hrow = S.h + grow * F;
#pragma unroll
      for (int jj = 0; jj < NS; ++jj) {
        const int hc = ntile * kHN + wn * WN + jj * 16 + (lane & 15);
        hrow[hc] = (uint8_t)__builtin_amdgcn_cvt_pk_fp8_f32(acc[i][jj][q] * f, 0.f, 0, false);
      }
      if (wn == 0 && (lane & 15) == 0) S.h_scale[grow * hblocks + ntile] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Gate/up GEMM + SwiGLU + h quantisation. Tile: BM rows x 128 h columns
// (128 gate + 128 up weight rows); wave (wm, wn) owns h columns
// [32 wn, 32 wn + 32) of rows [wm BM/WM, (wm + 1) BM/WM). A (activation rows,
// gathered through the permutation) is staged through LDS, double buffered
// and XOR-swizzled; each wave streams its own weight rows straight into a
// register ring PD K-steps deep. W4: MXFP4 weights (half the bytes per step,
// so the ring is twice as deep for the same bytes in flight; no channel
// scales).
// ---------------------------------------------------------------------------
template <int BM, int WM, int KTC, bool W4>
__global__ __launch_bounds__(kNWaves * WM * kWave) void gateup_fp8_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NTH = kNWaves * WM * kWave;
  constexpr int BMW = BM / WM;      // rows per wave
  constexpr int MS = BMW / 16;
  constexpr int WN = kHN / kNWaves; // 32 h columns per wave
  constexpr int NS = WN / 16;       // 2 h subtiles per wave
  constexpr int NB = 2 * NS;        // weight subtiles per wave (gate, up)
  constexpr int CH = BM * (kBK / 16);
  constexpr int CPT = (CH + NTH - 1) / NTH;
  constexpr int PD = !W4 ? prefetch_depth<BMW, 64>() : BMW <= 16 ? 6 : BMW <= 32 ? 4 : 3;
  // MXFP4 scales by quads where the K loop is unrolled over whole quads
  constexpr bool QS = W4 && KTC > 0 && KTC % 4 == 0;  // scales held per row (KT known)
  constexpr int KTS = QS ? KTC : 4;
  // MXFP4: a row's K step is half a 128-byte line; its two halves are loaded
  // together (after every second step, into the two slots just consumed), as
  // the FP8 fragment loads both halves of its line in one step
  constexpr bool PAIR = W4 && PD % 2 == 0;

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kBK];
  __shared__ float sxl[BM];
  __shared__ float red[kNWaves][BM];

  Tile te;
  if (!pick_tile<BM>(list, hdr->n_up, up_ntiles_max(c), te)) return;
  const int ntile = te.ntile;
  const int sid = te.gid >> 16, g = te.gid & 0xffff;
  const SetView S = set_view(c, sid);
  const int d = c.d, F = S.F;
  if (ntile >= F / kHN) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / kNWaves, wn = wave % kNWaves;
  const int rbase = wm * BMW;
  const uint8_t* a = static_cast<const uint8_t*>(c.a);

  // activation rows of this tile (gathered), their scales into LDS
  const uint8_t* a_src[CPT];
  int a_dst[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = tid + i * NTH;
    const int r = min(ch >> 3, BM - 1), c16 = ch & 7;
    const int grow = te.row0 + min(r, te.nrows - 1);
    const int src = min(max(S.row_src ? S.row_src[grow] / S.src_div : grow, 0), c.a_rows - 1);
    a_src[i] = a + (size_t)src * d + c16 * 16;
    a_dst[i] = swz(r, c16);
    if (ch < CH && c16 == 0) sxl[r] = c.a_scale[src];
  }
  // weight rows of this wave (and, MXFP4, their block scales)
  const size_t wrb = W4 ? d / 2 : d;  // weight bytes per row
  const uint8_t* w13 = S.w13 + (size_t)g * 2 * F * wrb;
  const uint8_t* b_src[NB];
  const uint8_t* e_src[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int hc = ntile * kHN + wn * WN + (j % NS) * 16 + (lane & 15);
    const int wrow = (j < NS) ? hc : F + hc;
    b_src[j] = w13 + (size_t)wrow * wrb + (lane >> 4) * 16;
    e_src[j] = W4 ? S.e13 + ((size_t)g * 2 * F + wrow) * (d / 32) + (QS ? 0 : lane >> 4) : nullptr;
  }
  // weight scales of this wave's columns, loaded now so that the epilogue
  // waits on no load (its stores sit under row guards, where a pending load
  // would make every store wait for all earlier ones)
  float sg[NS], su[NS];
#pragma unroll
  for (int jj = 0; jj < NS; ++jj) {
    const int hc = ntile * kHN + wn * WN + jj * 16 + (lane & 15);
    if constexpr (W4) {
      sg[jj] = 1.f;
      su[jj] = 1.f;
    } else {
      sg[jj] = S.s13[(size_t)g * 2 * F + hc];
      su[jj] = S.s13[(size_t)g * 2 * F + F + hc];
    }
  }

  v4f acc[MS][NB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Software pipeline, one K step (128 bytes of K) per stage:
  //   B (weights): register ring of PD steps; step kt's fragments are loaded
  //                right after step kt - PD has used the slot;
  //   A (rows):    LDS double buffer; step kt+1 is stored from registers loaded
  //                one full step earlier, then step kt+2 is loaded.
  // Every load is unconditional (the step index is clamped; tail re-loads hit
  // the cache), so the number of loads in flight is the same on every path and
  // the compiler's wait counts stay exact.
  const int KT = KTC > 0 ? KTC : d / kBK;  // KTC: K steps known at compile time
  v4i a_stage[CPT];
  BFrag<W4> bq[PD][NB];
  int srow[NB][KTS / 4];
  if constexpr (QS) {
#pragma unroll
    for (int j = 0; j < NB; ++j) load_scale_row<KTS>(srow[j], e_src[j], lane);
  }
#pragma unroll
  for (int s = 0; s < PD; ++s)
#pragma unroll
    for (int j = 0; j < NB; ++j) bq[s][j] = load_bfrag<W4, !QS>(b_src[j], e_src[j], min(s, KT - 1));
#pragma unroll
  for (int i = 0; i < CPT; ++i) a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i]);
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    if (CH % NTH == 0 || tid + i * NTH < CH)
      *reinterpret_cast<v4i*>(&lds_a[0][a_dst[i]]) = a_stage[i];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i] + min(1, KT - 1) * kBK);
  __syncthreads();

  // With KTC > 0 the loop is fully unrolled: no back edge, so the compiler's
  // wait counts are exact at every step.
#pragma unroll (KTC > 0 ? KTC : 1)
  for (int kt0 = 0; kt0 < KT; kt0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int kt = kt0 + s;
      if (kt < KT) {
        const int cur = kt & 1;
        if constexpr (QS) {
#pragma unroll
          for (int j = 0; j < NB; ++j) bq[s][j].s = scale_of_step<KTS>(srow[j], kt, lane);
        }
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const v8i af = lds_afrag(lds_a[cur] + rbase * kBK, i, lane);
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_w(af, bq[s][j], acc[i][j]);
        }
        // A for step kt+1 into the other buffer (its readers finished at the
        // barrier ending step kt-1), then fetch A for step kt+2
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          if (CH % NTH == 0 || tid + i * NTH < CH)
            *reinterpret_cast<v4i*>(&lds_a[cur ^ 1][a_dst[i]]) = a_stage[i];
        const int ka = min(kt + 2, KT - 1), kb = min(kt + PD, KT - 1);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i] + ka * kBK);
        if constexpr (PAIR) {
          if (s % 2 == 1) {  // kt0 is a multiple of the even PD: s has kt's parity
            const int kb0 = min(kt + PD - 1, KT - 1);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              bq[s - 1][j] = load_bfrag<W4, !QS>(b_src[j], e_src[j], kb0);
              bq[s][j] = load_bfrag<W4, !QS>(b_src[j], e_src[j], kb);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j) bq[s][j] = load_bfrag<W4, !QS>(b_src[j], e_src[j], kb);
        }
        __syncthreads();
        // keep each step's instructions in its step (bounds register pressure
        // of the unrolled loop)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  gateup_epilogue<BM, MS, NS>(acc, sxl, red, sg, su, rbase, wn, lane, te, S, ntile);
}



// Direct-to-LDS load of 16 bytes per lane (global_load_lds_dwordx4): a wave's
// 64 pieces land at lds_base + 16 lane. The tall-tile kernels stage tiles
// this way: a thread's piece lands at (the piece's 1 KiB block) + 16 lane, and
// a swizzle is applied by choosing which global chunk each lane fetches.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ inline void dma16(const uint8_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)lds_base, 16, 0, 0);
}
// The same with 4 bytes per lane (lane l's dword lands at lds_base + 4 l).
template <typename T>
__device__ inline void dma4(const T* src, T* lds_base) {
  static_assert(sizeof(T) == 4, "one dword per lane");
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left at their "no wait"
// maxima; gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS written by ordinary stores: waits for this wave's
// LDS operations (lgkmcnt) only, so global loads -- direct-to-LDS ones
// included, whose completion the caller waits for by vmcnt -- stay in flight
// (a release fence would wait for those too). The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(std::integral_constant<int, K>) for K = 0 .. N - 1 in order, so the
// body sees each K as a compile-time constant (a fully unrolled loop whose
// wait counts are template arguments).
template <class Fn, int... Ks>
__device__ inline void static_for_impl(Fn&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, class Fn>
__device__ inline void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Gate/up epilogue for the transposed product (weights as the MFMA A operand):
// lane l holds, for tile row rbase + 16 i + l % 16, the four consecutive h
// columns 16 jj + 4 (l / 16) + q of the wave's 16 NS (gate in acc[i][jj], up in
// acc[i][NS + jj]). SwiGLU, the row's block amax over the 128 h columns of the
// tile (the four lanes of a row, then the NWN waves of the row through LDS),
// its scale amax / 448, and the four E4M3 codes packed into one 32-bit store. The codes
// are h (1/s) by one multiply (silu_times, h_block_scale) and come from the
// packed float32 -> FP8 conversion, which rounds to nearest even and
// saturates exactly as e4m3_encode does for quotients of magnitude <= 448.
// The scales are read through accessors: sx(i) the x scale of row rbase +
// 16 i + lane % 16, sg(jj) / su(jj) the channel scales of gate / up columns
// c0 + 16 jj .. + 3 (ones for MXFP4 weights, which have none).
template <int BM, int MS, int NS, int NWN, class SX, class SG, class SU>
__device__ inline void gateup_epilogue_pp(v4f (&acc)[MS][2 * NS], SX sx, SG sg, SU su,
                                          float (*red)[BM], int rbase, int wn, int lane,
                                          const Tile& te, const SetView& S, int ntile) {
  constexpr int WN = NS * 16;
  const int F = S.F;
  const int c0 = wn * WN + 4 * (lane >> 4);
  // the rows' x scales and the columns' channel scales, read once before
  // the barrier below (a persistent caller's next tile may overwrite them
  // once every wave is past it) and up front (one wait for all of them)
  float sxv[MS];
  v4f sgv[NS], suv[NS];
#pragma unroll
  for (int jj = 0; jj < NS; ++jj) sgv[jj] = sg(jj), suv[jj] = su(jj);
#pragma unroll
  for (int i = 0; i < MS; ++i) sxv[i] = sx(i);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int r = rbase + i * 16 + (lane & 15);
    const float sxi = sxv[i];
    float m = 0.f;
#pragma unroll
    for (int jj = 0; jj < NS; ++jj) {
      const v4f sgj = sgv[jj], suj = suv[jj];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float gv = acc[i][jj][q] * sxi * sgj[q];
        const float hx = silu_times(gv, acc[i][NS + jj][q] * suj[q]);  // h / sx
        acc[i][jj][q] = hx;
        m = fmaxf(m, fabsf(hx));
      }
    }
    m = fmaxf(m, __shfl_xor(m, 16, kWave));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    if (lane < 16) red[wn][r] = m;
  }
  __syncthreads();
  const int hblocks = F / kHN;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int r = rbase + i * 16 + (lane & 15);
    if (r >= te.nrows) continue;
    float am = red[0][r];
#pragma unroll
    for (int ww = 1; ww < NWN; ++ww) am = fmaxf(am, red[ww][r]);
    const float s = h_block_scale(am, sxv[i]);
    const float f = sxv[i] * __builtin_amdgcn_rcpf(s);
    const size_t grow = (size_t)(te.row0 + r);
    int w[NS];
#pragma unroll
    for (int jj = 0; jj < NS; ++jj) {
      w[jj] = __builtin_amdgcn_cvt_pk_fp8_f32(acc[i][jj][0] * f, acc[i][jj][1] * f, 0, false);
      w[jj] = __builtin_amdgcn_cvt_pk_fp8_f32(acc[i][jj][2] * f, acc[i][jj][3] * f, w[jj], true);
    }
    if constexpr (NS == 4) {
      // The row's 64 bytes of this wave sit in its four lanes l % 16 + 16 q
      // as dwords 4 jj + q; a 4 x 4 transpose among them (two rounds of
      // pairwise exchanges, lanes l ^ 16 then l ^ 32) gives lane q dwords
      // 4 q .. 4 q + 3, stored as one 16-byte piece: an instruction writes
      // 16 rows x 64 contiguous bytes instead of 16 rows x 16.
      const int q = lane >> 4;
      {
        const int sa = (q & 1) ? w[0] : w[1], sb = (q & 1) ? w[2] : w[3];
        const int ra = __builtin_amdgcn_ds_swizzle(sa, 0x401F);  // lane ^ 16
        const int rb = __builtin_amdgcn_ds_swizzle(sb, 0x401F);
        if (q & 1) w[0] = ra, w[2] = rb; else w[1] = ra, w[3] = rb;
      }
      {
        const int sa = (q & 2) ? w[0] : w[2], sb = (q & 2) ? w[1] : w[3];
        const int ra = __shfl_xor(sa, 32, kWave), rb = __shfl_xor(sb, 32, kWave);
        if (q & 2) w[0] = ra, w[1] = rb; else w[2] = ra, w[3] = rb;
      }
      *reinterpret_cast<v4i*>(S.h + grow * F + ntile * kHN + wn * WN + 16 * q) =
          v4i{w[0], w[1], w[2], w[3]};
    } else if constexpr (NS == 2) {
      // The same with 32 bytes per row and wave (dwords 4 jj + q, jj < 2):
      // lane q ends with dwords 2 q and 2 q + 1, one 8-byte store.
      const int q = lane >> 4;
      const int keep = (q & 2) ? w[1] : w[0];
      const int got = __shfl_xor((q & 2) ? w[0] : w[1], 32, kWave);
      const int recv = __builtin_amdgcn_ds_swizzle(((q & 1) == ((q >> 1) & 1)) ? got : keep, 0x401F);
      const int lo = (q & 1) ? recv : ((q & 2) ? got : keep);
      const int hi = (q & 1) ? ((q & 2) ? keep : got) : recv;
      *reinterpret_cast<uint2*>(S.h + grow * F + ntile * kHN + wn * WN + 8 * q) =
          make_uint2((uint32_t)lo, (uint32_t)hi);
    } else {
      uint8_t* hrow = S.h + grow * F + ntile * kHN + c0;
#pragma unroll
      for (int jj = 0; jj < NS; ++jj) *reinterpret_cast<int*>(hrow + 16 * jj) = w[jj];
    }
    if (wn == 0 && lane < 16) S.h_scale[grow * hblocks + ntile] = s;
  }
}

// ---------------------------------------------------------------------------
// Gate/up GEMM for tall tiles (prefill), FP8 or MXFP4 weights (W4), ping-pong
// schedule.
// Tile BM rows x 128 h columns (256 weight rows: 128 gate, 128 up), 8 waves in
// two groups of four: group g owns rows [g BM/2, (g + 1) BM/2), wave wn of a
// group h columns [32 wn, 32 wn + 32). Each SIMD runs one wave of each group.
// Every K step is two phases per wave, LOAD (read the step's MFMA fragments
// from LDS into registers, write the next step's activation rows into LDS,
// issue later steps' global loads) and COMPUTE (the step's MFMAs, no memory
// access), separated by workgroup barriers; group 1 runs one phase behind
// group 0, so on every SIMD one wave loads while the other computes and the
// matrix core is fed from registers without waiting on LDS.
//
// Operand staging: activation rows (gathered through the permutation) are
// loaded into registers two steps ahead and written into one of two LDS
// stages a step ahead; weight rows go straight from global memory into one of
// NBS LDS stages D = NBS - 1 steps ahead (direct-to-LDS loads; MXFP4 rows of
// 64 bytes per K step, 16 to a 1 KiB block, their E8M0 scales in an LDS tile
// filled once per workgroup, one dword of padding per row). Phase by phase
// the two groups' reads of a stage finish before either overwrites it:
//   phase 2 kt:     group 0 LOAD(kt)    group 1 COMPUTE(kt - 1)
//   phase 2 kt + 1: group 0 COMPUTE(kt) group 1 LOAD(kt)
// LOAD(kt) reads A stage kt % 2 and B stage kt % NBS, writes A stage
// (kt + 1) % 2 and loads B stage (kt + D) % NBS, both last read in phase
// 2 kt - 1; each wave waits for its own part of B step kt + 1 before the
// barrier that ends phase 2 kt + 1, the last one before that step is first
// read. The K loop is fully unrolled, so every wait count is exact. After the
// loop the A stages hold the epilogue's row maxima.
// ---------------------------------------------------------------------------
template <int BM, int KTC, int NBS, bool W4>
__global__ __launch_bounds__(8 * kWave) void gateup_fp8_pp_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NW = 8;
  constexpr int BMW = BM / 2, MS = BMW / 16;
  constexpr int NS = 2, NB = 2 * NS;
  constexpr int BROWS = 2 * kHN;                 // weight rows per tile
  constexpr int KB = kstep_bytes<W4>();          // weight bytes per row and K step
  constexpr int NAD = BM * kBK / 1024 / NW;      // A pieces (16 B) per thread per step
  constexpr int NBD = BROWS * KB / 1024 / NW;    // B pieces per thread per step
  constexpr int D = NBS - 1;                     // weight steps loaded ahead
  constexpr int SSC = W4 ? BROWS * (KTC + 1) : 1;  // MXFP4 scale tile (dwords)
  static_assert(BM * kBK % (1024 * NW) == 0, "A tile must split into whole wave loads");
  static_assert(KTC >= NBS, "the pipeline holds NBS K steps");
  static_assert(NBS >= 3 && NBS <= 4, "three or four weight stages");
  static_assert(kNWaves * BM * 4 <= BM * kBK, "row maxima fit in an A stage");
  static_assert(!W4 || KTC % 4 == 0, "MXFP4 scales are held per row in K-step quads");
  // the x and channel scales stay in LDS when it has room beside the stages,
  // else in registers
  constexpr bool SCL =
      2 * BM * kBK + NBS * BROWS * KB + (W4 ? 4 * SSC : 0) + (BM + BROWS) * 4 <= 163840;

  // one LDS variable per stage: the compiler tells distinct variables apart,
  // so a read of one stage does not wait for the direct-to-LDS loads still in
  // flight into the others (slices of one array it cannot separate, and it
  // would drain every weight load before each LOAD phase)
  __shared__ __attribute__((aligned(1024))) uint8_t a0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[BROWS * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[BROWS * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b2[BROWS * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b3[NBS > 3 ? BROWS * KB : 16];
  __shared__ int ssc[SSC];
  __shared__ float sxl[SCL ? BM : 1];
  __shared__ __attribute__((aligned(16))) float s13l[(SCL && !W4) ? BROWS : 1];

  Tile te;
  if (!pick_tile<BM>(list, hdr->n_up, up_ntiles_max(c), te)) return;
  const int ntile = te.ntile;
  const int sid = te.gid >> 16, g = te.gid & 0xffff;
  const SetView S = set_view(c, sid);
  const int d = c.d, F = S.F;
  if (ntile >= F / kHN) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / kNWaves, wn = wave % kNWaves;
  const int rbase = grp * BMW;
  const uint8_t* a = static_cast<const uint8_t*>(c.a);
  auto src_row = [&](int r) {  // activation row of tile row r
    const int grow = te.row0 + min(r, te.nrows - 1);
    return min(max(S.row_src ? S.row_src[grow] / S.src_div : grow, 0), c.a_rows - 1);
  };

  // A piece i of this thread: tile row 8 (NAD wave + i) + lane / 8, stored at
  // (its 1 KiB block) + 16 lane, the swizzle applied by the source chunk
  const uint8_t* asrc[NAD];
#pragma unroll
  for (int i = 0; i < NAD; ++i) {
    const int r = 8 * (NAD * wave + i) + (lane >> 3);
    const int cch = (lane & 7) ^ (r & 7);
    asrc[i] = a + (size_t)src_row(r) * d + cch * 16;
  }
  // B piece i (rows 0..127 gate, 128..255 up): FP8 weight-tile row
  // 8 (NBD wave + i) + lane / 8, the same layout; MXFP4 16 rows of 64 bytes
  // per 1 KiB block, row 16 (NBD wave + i) + lane / 4, its 16-byte chunk q
  // stored at chunk q ^ ((row / 2) % 4): a 16-byte-per-lane LDS read is served
  // 8 lanes at a time from a 128-byte bank window, and any 8 consecutive rows
  // of a fragment read then fall in 8 different 16-byte slots of it (with
  // q ^ ((row / 4) % 4) rows r and r + 2 shared a slot: 2-way bank conflicts)
  const size_t wrb = W4 ? d / 2 : d;  // weight bytes per row
  const uint8_t* w13 = S.w13 + (size_t)g * 2 * F * wrb;
  auto wrow_of = [&](int rr) { return (rr < kHN) ? ntile * kHN + rr : F + ntile * kHN + (rr - kHN); };
  const uint8_t* bsrc[NBD];
#pragma unroll
  for (int i = 0; i < NBD; ++i) {
    if constexpr (W4) {
      const int rr = 16 * (NBD * wave + i) + (lane >> 2);
      const int cch = (lane & 3) ^ ((rr >> 1) & 3);
      bsrc[i] = w13 + (size_t)wrow_of(rr) * wrb + cch * 16;
    } else {
      const int rr = 8 * (NBD * wave + i) + (lane >> 3);
      const int cch = (lane & 7) ^ (rr & 7);
      bsrc[i] = w13 + (size_t)wrow_of(rr) * wrb + cch * 16;
    }
  }
  // MXFP4: the tile's E8M0 scales into LDS (published by the prologue's barrier)
  if constexpr (W4)
    fill_scale_tile<KTC, BROWS, 8 * kWave>(
        ssc, [&](int r) { return S.e13 + ((size_t)g * 2 * F + wrow_of(r)) * (d / 32); }, tid);
  // the epilogue's x scales and channel scales (FP8), loaded now
  const float* s13 = W4 ? nullptr : S.s13 + (size_t)g * 2 * F;
  float sxr[SCL ? 1 : MS];
  v4f sgr[(SCL || W4) ? 1 : NS], sur[(SCL || W4) ? 1 : NS];
  if constexpr (SCL) {
    if (tid < BM) sxl[tid] = c.a_scale[src_row(tid)];
    if constexpr (!W4) {
      if (tid < BROWS) s13l[tid] = s13[wrow_of(tid)];
    }
  } else {
#pragma unroll
    for (int i = 0; i < MS; ++i) sxr[i] = c.a_scale[src_row(rbase + i * 16 + (lane & 15))];
    if constexpr (!W4) {
      const float* sc = s13 + ntile * kHN + wn * 32 + 4 * (lane >> 4);
#pragma unroll
      for (int jj = 0; jj < NS; ++jj) {
        sgr[jj] = *reinterpret_cast<const v4f*>(sc + 16 * jj);
        sur[jj] = *reinterpret_cast<const v4f*>(sc + F + 16 * jj);
      }
    }
  }

  v4i ra[2][NAD];  // activation rows of two K steps in flight
  auto lda = [&](int kt, int slot) {
#pragma unroll
    for (int i = 0; i < NAD; ++i) ra[slot][i] = *reinterpret_cast<const v4i*>(asrc[i] + kt * kBK);
  };
  auto sta = [&](int slot, uint8_t* ad) {
#pragma unroll
    for (int i = 0; i < NAD; ++i)
      *reinterpret_cast<v4i*>(ad + (NAD * wave + i) * 1024 + lane * 16) = ra[slot][i];
  };
  auto ldb = [&](int kt, uint8_t* bd) {
#pragma unroll
    for (int i = 0; i < NBD; ++i) dma16(bsrc[i] + kt * KB, bd + (NBD * wave + i) * 1024);
  };
  auto astage = [&](int kt) { return (kt & 1) ? a1 : a0; };
  auto bstage = [&](int kt) {
    const int m = kt % NBS;
    return m == 0 ? b0 : m == 1 ? b1 : m == 2 ? b2 : b3;
  };

  // prologue: A(0), B(0) .. B(D - 2), A(1), B(D - 1) (the order the wait
  // counts of pipeline.h assume; scheduling barriers keep the compiler from
  // reordering the groups); A(0) into its stage, B(0) landed
  lda(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s + 1 < D; ++s) ldb(s, bstage(s));
  __builtin_amdgcn_sched_barrier(0);
  lda(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  ldb(D - 1, bstage(D - 1));
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<(D - 1) * NBD + NAD + NBD>();
  sta(0, a0);
  wait_vmcnt<(D - 2) * NBD + NAD + NBD>();
  lds_barrier();  // publishes A(0) and B(0)
  if (grp == 1) __builtin_amdgcn_s_barrier();  // group 1 one phase behind
  __builtin_amdgcn_sched_barrier(0);

  v4f acc[MS][NB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  static_for<KTC>([&](auto ktc) {
    constexpr int kt = decltype(ktc)::value;
    // ---- LOAD(kt) ----
    if constexpr (kt + 1 < KTC) {
      wait_vmcnt<pp_after_a(kt, D, KTC, NAD, NBD)>();  // A(kt + 1) in registers
      sta((kt + 1) & 1, astage(kt + 1));
    }
    BFrag<W4> bf[NB];
    v8i af[MS];
    {
      const uint8_t* bs = bstage(kt);
      const uint8_t* as = astage(kt);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int row0 = (j < NS) ? wn * 32 + j * 16 : kHN + wn * 32 + (j - NS) * 16;
        if constexpr (W4) {
          const int r = row0 + (lane & 15);
          bf[j].w = *reinterpret_cast<const v4i*>(bs + r * KB + (((lane >> 4) ^ ((r >> 1) & 3)) << 4));
          bf[j].s = scale_from_tile<KTC>(ssc, r, kt, lane);
        } else {
          bf[j] = lds_afrag(bs + row0 * kBK, 0, lane);
        }
      }
#pragma unroll
      for (int i = 0; i < MS; ++i) af[i] = lds_afrag(as + rbase * kBK, i, lane);
    }
    if constexpr (kt + 2 < KTC) lda(kt + 2, kt & 1);
    __builtin_amdgcn_sched_barrier(0);  // A before B: the order the counts assume
    if constexpr (kt + D < KTC) ldb(kt + D, bstage(kt + D));
    // this wave's part of B(kt + 1) lands before the barrier ending phase
    // 2 kt + 1: group 1 waits here, group 0 after its COMPUTE(kt)
    constexpr int wb = (kt + 1 < KTC) ? pp_after_b(kt, D, KTC, NAD, NBD) : 0;
    if (grp == 1) wait_vmcnt<wb>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- COMPUTE(kt) ----
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mfma_wt(bf[j], af[i], acc[i][j]);
    if constexpr (W4) {
      // the block-scaled MFMAs stay in their phase (left free, the scheduler
      // defers them and runs out of registers)
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    if (grp == 0) wait_vmcnt<wb>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  });
  if (grp == 0) __builtin_amdgcn_s_barrier();  // both groups aligned again
  wait_vmcnt<0>();
  float(*red)[BM] = reinterpret_cast<float(*)[BM]>(a0);
  const v4f one = v4f{1.f, 1.f, 1.f, 1.f};  // MXFP4: no channel scales
  if constexpr (SCL) {
    const int c0 = wn * 32 + 4 * (lane >> 4);
    gateup_epilogue_pp<BM, MS, NS, kNWaves>(
        acc, [&](int i) { return sxl[rbase + i * 16 + (lane & 15)]; },
        [&](int jj) { return W4 ? one : *reinterpret_cast<const v4f*>(&s13l[c0 + 16 * jj]); },
        [&](int jj) { return W4 ? one : *reinterpret_cast<const v4f*>(&s13l[kHN + c0 + 16 * jj]); },
        red, rbase, wn, lane, te, S, ntile);
  } else {
    gateup_epilogue_pp<BM, MS, NS, kNWaves>(
        acc, [&](int i) { return sxr[i]; }, [&](int jj) { return W4 ? one : sgr[jj]; },
        [&](int jj) { return W4 ? one : sur[jj]; }, red, rbase, wn, lane, te, S, ntile);
  }
}

// Weight stages of the ping-pong gate/up kernel: four where the LDS holds them
// (128 rows; MXFP4, whose stages are half the bytes), three at 192 rows of FP8.
template <int BM, bool W4>
constexpr int pp_weight_stages() { return (W4 || BM <= 128) ? 4 : 3; }

// Side work of one K step of the four-wave gate/up kernel, at most two items
// per MFMA slot (m = 0 .. NSLOT - 1). Global loads sit in every third slot,
// each right after the LDS write that frees its registers (activation piece
// p: write in slot 3 p, reload in 3 p + 1; then weight piece q likewise at
// 3 (NA + q)), because the four waves reach the same slot together and
// bunched loads back up the CU's address queue, which stalls the loading
// wave's MFMAs behind them. LDS fragment reads fill the rest, two to a slot
// where needed: B fragment j (two reads) only after slot MS j + MS - 1, its
// last MFMA (except the last fragment, whose registers alternate), A
// fragment halves anywhere.
enum IwOp { kIwNone, kIwStA, kIwLdA, kIwStB, kIwLdB, kIwRdA, kIwRdB };
template <int NSLOT>
struct IwSlots {
  int op[2][NSLOT];
  int arg[2][NSLOT];
};
template <int NSLOT, int NA, int NBL, int MS, int NBF>
constexpr IwSlots<NSLOT> iw_slots() {
  IwSlots<NSLOT> t{};
  for (int h = 0; h < 2; ++h)
    for (int m = 0; m < NSLOT; ++m) t.op[h][m] = kIwNone, t.arg[h][m] = 0;
  for (int p = 0; p < NA + NBL; ++p) {
    const bool a = p < NA;
    t.op[0][3 * p] = a ? kIwStA : kIwStB, t.arg[0][3 * p] = a ? p : p - NA;
    t.op[0][3 * p + 1] = a ? kIwLdA : kIwLdB, t.arg[0][3 * p + 1] = a ? p : p - NA;
  }
  // a read goes to the earliest slot at or after lo with room: an empty
  // slot, else the second place of a slot that holds no global load
  auto place = [&](int lo, int op, int arg) {
    for (int pass = 0; pass < 2; ++pass)
      for (int m = lo; m < NSLOT; ++m) {
        if (pass == 0 && t.op[0][m] == kIwNone) {
          t.op[0][m] = op, t.arg[0][m] = arg;
          return;
        }
        if (pass == 1 && t.op[1][m] == kIwNone && t.op[0][m] != kIwLdA && t.op[0][m] != kIwLdB) {
          t.op[1][m] = op, t.arg[1][m] = arg;
          return;
        }
      }
  };
  for (int f = 0; f < 2 * NBF; ++f) {
    const int j = f / 2;
    place((j + 1 < NBF) ? MS * j + MS : 0, kIwRdB, f);
  }
  for (int f = 0; f < 2 * MS; ++f) place(0, kIwRdA, f);
  return t;
}
template <int NSLOT, int NA, int NBL, int MS, int NBF>
constexpr bool iw_slots_complete() {
  constexpr IwSlots<NSLOT> t = iw_slots<NSLOT, NA, NBL, MS, NBF>();
  int n[7] = {0, 0, 0, 0, 0, 0, 0};
  for (int h = 0; h < 2; ++h)
    for (int m = 0; m < NSLOT; ++m) ++n[t.op[h][m]];
  return 3 * (NA + NBL) <= NSLOT && n[kIwStA] == NA && n[kIwLdA] == NA && n[kIwStB] == NBL &&
         n[kIwLdB] == NBL && n[kIwRdA] == 2 * MS && n[kIwRdB] == 2 * NBF;
}

// ---------------------------------------------------------------------------
// Gate/up GEMM for tall tiles, one wave per SIMD. Tile BM rows x 128 h
// columns (256 weight rows), 4 waves: wave (wm, wn) owns rows
// [wm BM/2, (wm + 1) BM/2) and h columns [64 wn, 64 wn + 64) (weight rows
// [64 wn, +64) gate and 128 + [64 wn, +64) up). A wave's 96 x 128
// accumulator tile (192 registers per lane) needs more registers than two
// waves per SIMD leave each, and reads 7/10 of the LDS bytes per MFMA of the
// ping-pong kernel's 96 x 64 tiles; the ping-pong kernel's K steps are bound
// by their LDS reads, this one's by its MFMAs.
//
// Each wave overlaps its own LDS traffic with its MFMAs: while the MFMAs of
// step kt run (B fragment by B fragment), it reads step kt + 1's fragments
// (each B fragment's registers right after the last MFMA that uses them; the
// A fragments into a second set), writes step kt + 2's operand rows into the
// stages step kt's rows left, and issues later steps' global loads.
// One workgroup barrier per step, at its end: by then every wave has read
// step kt + 1's fragments (so the stages of step kt + 1 may be overwritten
// from step kt + 1 on) and written its part of step kt + 2 (read during step
// kt + 1).
//
// Operand staging: both operands go through registers -- weight rows loaded
// two steps before they are written into LDS (two register sets), activation
// rows one step (one set; mostly L2 hits) -- and are written two steps before
// their fragments are computed with (two LDS stages each).
// Direct-to-LDS loads would save the registers and the LDS writes, but each
// stalls its (only) wave's instruction issue for tens of cycles, and here
// that wave also issues the MFMAs. Activation rows are gathered through the
// permutation; MXFP4 weights' E8M0 scales sit in an LDS tile filled once per
// workgroup.
// ---------------------------------------------------------------------------
template <int BM, int KTC, bool W4>
__global__ __launch_bounds__(4 * kWave) void gateup_fp8_iw_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NW = 4;
  constexpr int BMW = BM / 2, MS = BMW / 16;
  constexpr int NS = 4, NB = 2 * NS;             // gate and up fragments per wave
  constexpr int BROWS = 2 * kHN;                 // weight rows per tile
  constexpr int KB = kstep_bytes<W4>();          // weight bytes per row and K step
  constexpr int NAD = BM * kBK / 1024 / NW;      // A pieces (16 B) per thread per step
  constexpr int NBD = BROWS * KB / 1024 / NW;    // B pieces per thread per step
  constexpr int SSC = W4 ? BROWS * (KTC + 1) : 1;  // MXFP4 scale tile (dwords)
  constexpr int NSP = W4 ? scale_pieces<KTC, BROWS, NW * kWave>() : 1;
  constexpr int RPB = W4 ? 16 : 8;  // weight rows per 1 KiB block
  static_assert(BM * kBK % (1024 * NW) == 0, "A tile must split into whole wave loads");
  static_assert(KTC >= 4, "the prologue loads four steps");
  static_assert(!W4 || KTC % 4 == 0, "MXFP4 scales are held per row in K-step quads");
  static_assert(NBD * RPB * NW == BROWS && NBD * RPB <= kHN / 2, "a wave's pieces in one half");
  static_assert(2 * BM * kBK + 2 * BROWS * KB + (W4 ? 4 * SSC : 0) + (3 * BM + BROWS) * 4 <= 163840,
                "stages and scales fit the LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t a0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[BROWS * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[BROWS * KB];
  __shared__ int ssc[SSC];
  __shared__ float sxl[BM];
  __shared__ __attribute__((aligned(16))) float s13l[W4 ? 1 : BROWS];
  __shared__ float red[2][BM];  // the epilogue's row maxima

  // (tid and lane are re-declared unknown to the compiler at each tile, so
  // addresses derived from them are computed per tile: hoisted out of the
  // tile loop they would stay live across the K loop, which needs every
  // register)
  int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int rbase = wm * BMW;
  const int d = c.d;
  const uint8_t* a = static_cast<const uint8_t*>(c.a);

  // The workgroup's tiles: slots slot, slot + sstep, ... of its XCD's items
  // (pick_tile's order), skipping N tiles past a set's width.
  const int NT = up_ntiles_max(c), n_ent = hdr->n_up;
  const int xcd = blockIdx.x % kXcds, sstep = gridDim.x / kXcds;
  auto next_tile = [&](int& sl, Tile& t) {
    for (; pick_tile_at<BM>(list, n_ent, NT, xcd, sl, t); sl += sstep)
      if (t.ntile < ((t.gid >> 16) ? c.set[1].F : c.set[0].F) / kHN) return true;
    return false;
  };

  // Per-tile state. B piece i: FP8 weight-tile row RPB (NBD wave + i) +
  // lane / 8 (rows 0..127 gate, 128..255 up), chunks swizzled as the A
  // tile's; MXFP4 rows of 64 bytes, RPB = 16 to a block, row 16 (NBD wave + i)
  // + lane / 4, its chunk q stored at q ^ ((row / 2) % 4) (conflict-free
  // 16-byte fragment reads). A wave's pieces lie in one half (64 rows) and
  // share the chunk, so piece i is piece 0 plus i RPB rows: one per-lane
  // offset, the rest uniform. A piece i: tile row 8 (NAD wave + i) + lane / 8,
  // stored at (its 1 KiB block) + 16 lane, the swizzle applied by the source
  // chunk (32-bit offsets from the activation base).
  // (only derived values live across the K loop: the tile, its weights,
  // scale rows and output pointers -- not the whole set view)
  Tile te;
  int F = 0, sxrow = 0;
  size_t wrb = 0;
  const uint8_t* w13 = nullptr;   // the group's gate/up weight rows
  const uint8_t* e13g = nullptr;  // MXFP4: their scale rows
  const float* s13g = nullptr;    // FP8: their channel scales
  uint8_t* h_out = nullptr;
  float* hs_out = nullptr;
  uint32_t boff = 0, aoff[NAD];
  auto wrow_of = [&](int rr) { return (rr < kHN) ? te.ntile * kHN + rr : F + te.ntile * kHN + (rr - kHN); };
  auto setup = [&]() {
    const SetView S = set_view(c, te.gid >> 16);
    const int g = te.gid & 0xffff;
    F = S.F;
    wrb = W4 ? d / 2 : d;
    w13 = S.w13 + (size_t)g * 2 * F * wrb;
    if constexpr (W4)
      e13g = S.e13 + (size_t)g * 2 * F * (d / 32);
    else
      s13g = S.s13 + (size_t)g * 2 * F;
    h_out = S.h;
    hs_out = S.h_scale;
    const int rr = RPB * NBD * wave + (W4 ? (lane >> 2) : (lane >> 3));
    const int cch = W4 ? ((lane & 3) ^ ((rr >> 1) & 3)) : ((lane & 7) ^ (rr & 7));
    boff = (uint32_t)wrow_of(rr) * (uint32_t)wrb + (cch << 4);
    // the permutation's entries in one batch (row NAD: the x-scale row of
    // thread tid)
    int r[NAD + 1], src[NAD + 1];
#pragma unroll
    for (int i = 0; i < NAD; ++i) r[i] = 8 * (NAD * wave + i) + (lane >> 3);
    r[NAD] = min(tid, BM - 1);
    gather_rows(te, S, c.a_rows, r, src);
#pragma unroll
    for (int i = 0; i < NAD; ++i)
      aoff[i] = (uint32_t)src[i] * (uint32_t)d + (((lane & 7) ^ (r[i] & 7)) << 4);
    sxrow = src[NAD];
  };
  auto bsrc = [&](int kt, int i) { return w13 + (size_t)i * RPB * wrb + kt * KB + boff; };

  // operand rows in registers from their load to their LDS write: weight
  // rows two steps ahead (set kt & 1 holds step kt's), activation rows one
  // (one set; they mostly come from the L2)
  v4i ra[NAD], rb[2][NBD];
  auto lda = [&](v4i (&r)[NAD], int kt) {
#pragma unroll
    for (int i = 0; i < NAD; ++i) r[i] = *reinterpret_cast<const v4i*>(a + aoff[i] + kt * kBK);
  };
  auto ldb = [&](int kt, int slot) {
#pragma unroll
    for (int i = 0; i < NBD; ++i) rb[slot][i] = *reinterpret_cast<const v4i*>(bsrc(kt, i));
  };
  auto astage = [&](int kt) { return (kt & 1) ? a1 : a0; };
  auto bstage = [&](int kt) { return (kt & 1) ? b1 : b0; };
  // Fragments are read in halves, one LDS instruction each: A fragment i of
  // a stage is two 16-byte reads at rows rbase + 16 i + lane % 16; B fragment
  // j (rows 0..63 of the wave's 128: gate, 64..127: up) two reads (FP8) or
  // the codes and the scale byte (MXFP4).
  auto brow0 = [&](int j) { return (j < NS) ? wn * 64 + j * 16 : kHN + wn * 64 + (j - NS) * 16; };
  auto rda_half = [&](v8i& f, const uint8_t* as, int i, int h) {
    const int r = rbase + i * 16 + (lane & 15);
    const v4i v = *reinterpret_cast<const v4i*>(as + swz(r, 4 * h + (lane >> 4)));
    if (h == 0) f.lo = v; else f.hi = v;
  };
  auto rdb_half = [&](BFrag<W4>& f, const uint8_t* bs, int j, int h, int kt) {
    const int r = brow0(j) + (lane & 15);
    if constexpr (W4) {
      if (h == 0)
        f.w = *reinterpret_cast<const v4i*>(bs + r * KB + (((lane >> 4) ^ ((r >> 1) & 3)) << 4));
      else
        f.s = scale_from_tile<KTC>(ssc, r, kt, lane);
    } else {
      const v4i v = *reinterpret_cast<const v4i*>(bs + swz(r, 4 * h + (lane >> 4)));
      if (h == 0) f.lo = v; else f.hi = v;
    }
  };

  // A tile's first loads: activations and weights of steps 0 and 1 straight
  // into their LDS stages (the same layout the register path writes; outside
  // the K loop a direct-to-LDS load's issue stall costs nothing), its x and
  // channel scales (MXFP4: its scale tile's pieces) into registers. Issued
  // for the next tile before the current one's epilogue, which uses none of
  // the stages, so they land meanwhile.
  v4i scp[NSP];
  float sxv = 0.f, s13v = 0.f;
  auto issue_first = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < NAD; ++i)
        dma16(a + aoff[i] + s * kBK, astage(s) + (NAD * wave + i) * 1024);
#pragma unroll
      for (int i = 0; i < NBD; ++i) dma16(bsrc(s, i), bstage(s) + (NBD * wave + i) * 1024);
    }
    sxv = c.a_scale[sxrow];
    if constexpr (W4)
      load_scale_pieces<KTC, BROWS, NW * kWave>(
          scp, [&](int r) { return e13g + (size_t)wrow_of(r) * (d / 32); }, tid);
    else
      s13v = s13g[wrow_of(tid)];  // 256 threads, 256 weight rows
  };

  int slot = blockIdx.x / kXcds;
  if (!next_tile(slot, te)) return;
  setup();
  issue_first();
  for (;;) {
    asm volatile("" : "+v"(tid), "+v"(lane));
    // prologue: steps 0 and 1 landed in LDS (this wave's part: every load
    // it issued, the previous tile's epilogue stores included), the scales
    // into LDS, weights of steps 2 and 3 and activations of step 2 loaded,
    // step 0's fragments read
    wait_vmcnt<0>();
    if (tid < BM) sxl[tid] = sxv;
    if constexpr (W4)
      store_scale_pieces<KTC, BROWS, NW * kWave>(ssc, scp, tid);
    else
      s13l[tid] = s13v;
    __builtin_amdgcn_sched_barrier(0);
    lda(ra, 2);
    ldb(2, 0);
    ldb(3, 1);
    lds_barrier();  // publishes steps 0 and 1 and the scales

    // B fragment NB - 1 is used by a step's last MFMA, so it alternates
    // between two register sets; the others are re-read into their own
    // registers after their step's last MFMA with them
    BFrag<W4> bf[NB + 1];
    v8i af[2][MS];
    auto bslot = [&](int j, int kt) { return (j == NB - 1 && (kt & 1)) ? NB : j; };
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      rdb_half(bf[j], b0, j, 0, 0);
      rdb_half(bf[j], b0, j, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      rda_half(af[0][i], a0, i, 0);
      rda_half(af[0][i], a0, i, 1);
    }
    lds_barrier();  // every wave has read stage 0, which step 0 overwrites

    v4f acc[MS][NB];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);

    constexpr int NSLOT = NB * MS;  // MFMAs per step
    static_assert(iw_slots_complete<NSLOT, NAD, NBD, MS, NB>(), "a step's side work fits its slots");
    constexpr IwSlots<NSLOT> slots = iw_slots<NSLOT, NAD, NBD, MS, NB>();

    static_for<KTC>([&](auto ktc) {
      constexpr int kt = decltype(ktc)::value;
      constexpr int cur = kt & 1, nxt = cur ^ 1;
      static_for<NSLOT>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int j = m / MS, i = m % MS;
        acc[i][j] = mfma_wt(bf[bslot(j, kt)], af[cur][i], acc[i][j]);
        static_for<2>([&](auto hc) {
          constexpr int op = slots.op[decltype(hc)::value][m], q = slots.arg[decltype(hc)::value][m];
          if constexpr (op == kIwStA) {  // over step kt's rows, read in step kt - 1
            if constexpr (kt + 2 < KTC)
              *reinterpret_cast<v4i*>(astage(kt) + (NAD * wave + q) * 1024 + lane * 16) = ra[q];
          } else if constexpr (op == kIwStB) {
            if constexpr (kt + 2 < KTC)
              *reinterpret_cast<v4i*>(bstage(kt) + (NBD * wave + q) * 1024 + lane * 16) = rb[cur][q];
          } else if constexpr (op == kIwLdA) {
            if constexpr (kt + 3 < KTC)
              ra[q] = *reinterpret_cast<const v4i*>(a + aoff[q] + (kt + 3) * kBK);
          } else if constexpr (op == kIwLdB) {
            if constexpr (kt + 4 < KTC)
              rb[cur][q] = *reinterpret_cast<const v4i*>(bsrc(kt + 4, q));
          } else if constexpr (op == kIwRdA) {
            if constexpr (kt + 1 < KTC) rda_half(af[nxt][q / 2], astage(kt + 1), q / 2, q % 2);
          } else if constexpr (op == kIwRdB) {
            if constexpr (kt + 1 < KTC)
              rdb_half(bf[bslot(q / 2, kt + 1)], bstage(kt + 1), q / 2, q % 2, kt + 1);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      // with the barrier's LDS wait: step kt + 2 is written and step kt + 1's
      // fragments are in registers (the compiler waits for each register load
      // before the LDS write that uses it)
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    });

    // the accumulators as of the last step (an empty use here keeps the
    // MFMAs, whose results only the epilogue reads, from being moved past
    // the branch below into the epilogue, with every step's fragments kept
    // alive until then)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+a"(acc[i][j]));
    // the next tile's first loads, then this tile's epilogue (its scales
    // stay in LDS until the next prologue's first barrier; the stages are
    // free since the last step's barrier)
    const Tile tc = te;
    SetView Sc;  // what the epilogue reads of the set
    Sc.h = h_out;
    Sc.h_scale = hs_out;
    Sc.F = F;
    int sn = slot + sstep;
    Tile tn;
    const bool more = next_tile(sn, tn);
    if (more) {
      te = tn;
      slot = sn;
      setup();
      issue_first();
    }
    const v4f one = v4f{1.f, 1.f, 1.f, 1.f};  // MXFP4: no channel scales
    const int c0 = wn * 64 + 4 * (lane >> 4);
    gateup_epilogue_pp<BM, MS, NS, 2>(
        acc, [&](int i) { return sxl[rbase + i * 16 + (lane & 15)]; },
        [&](int jj) { return W4 ? one : *reinterpret_cast<const v4f*>(&s13l[c0 + 16 * jj]); },
        [&](int jj) { return W4 ? one : *reinterpret_cast<const v4f*>(&s13l[kHN + c0 + 16 * jj]); },
        red, rbase, wn, lane, tc, Sc, tc.ntile);
    if (!more) break;
    // the epilogue read sxl and s13l before its barrier; every wave is past it
  }
}

// ---------------------------------------------------------------------------
// Down GEMM with per-(row, 128-K block) h scales. Tile: BM rows x 256 output
// channels; wave (wm, wn) owns channels [64 wn, 64 wn + 64) of rows
// [wm BM/WM, (wm + 1) BM/WM). Each 128-wide K step is one h block: its MFMA
// partial is scaled by s_h[row][block] and accumulated.
// ---------------------------------------------------------------------------
template <int BM, int WM, int KTC, bool W4>
__global__ __launch_bounds__(kNWaves * WM * kWave) void down_fp8_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NTH = kNWaves * WM * kWave;
  constexpr int BMW = BM / WM;
  constexpr int MS = BMW / 16;
  constexpr int NB = 4;  // 16-channel subtiles per wave
  constexpr int CH = BM * (kBK / 16);
  constexpr int CPT = (CH + NTH - 1) / NTH;
  constexpr int PD = W4 ? 4 : prefetch_depth<BMW, 32>();
  constexpr bool PAIR = W4;  // both halves of a row's line together (gate/up kernel)

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kBK];
  __shared__ float hsl[2][BM];

  Tile te;
  if (!pick_tile<BM>(list, hdr->n_down, down_ntiles(c.d), te)) return;
  const int ntile = te.ntile;
  const int sid = te.gid >> 16, g = te.gid & 0xffff;
  const SetView S = set_view(c, sid);
  const int d = c.d, F = S.F, hblocks = F / kHN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / kNWaves, wn = wave % kNWaves;
  const int rbase = wm * BMW;

  const uint8_t* a_src[CPT];
  int a_dst[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = tid + i * NTH;
    const int r = min(ch >> 3, BM - 1), c16 = ch & 7;
    const int grow = te.row0 + min(r, te.nrows - 1);
    a_src[i] = S.h + (size_t)grow * F + c16 * 16;
    a_dst[i] = swz(r, c16);
  }
  // per-row h scales: thread r < BM fetches s_h[row r][kt]
  const float* hs_src = S.h_scale + (size_t)(te.row0 + min(tid, te.nrows - 1)) * hblocks;

  const size_t wrb = W4 ? F / 2 : F;  // weight bytes per row
  const uint8_t* w2 = S.w2 + (size_t)g * d * wrb;
  const uint8_t* b_src[NB];
  const uint8_t* e_src[NB];
  int mcol[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    mcol[j] = ntile * kDownBN + wn * (NB * 16) + j * 16 + (lane & 15);
    const size_t row = min(mcol[j], d - 1);
    b_src[j] = w2 + row * wrb + (lane >> 4) * 16;
    e_src[j] = W4 ? S.e2 + ((size_t)g * d + row) * (F / 32) + (lane >> 4) : nullptr;
  }
  // channel scales, loaded now so that the epilogue waits on no load
  float s2v[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) s2v[j] = W4 ? 1.f : S.s2[(size_t)g * d + min(mcol[j], d - 1)];

  v4f acc[MS][NB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Same pipeline as the gate/up GEMM; the per-row h scale of step kt+1 rides
  // with its A tile.
  const int KT = KTC > 0 ? KTC : F / kBK;  // KTC: K steps known at compile time
  v4i a_stage[CPT];
  float hs_stage;
  BFrag<W4> bq[PD][NB];
#pragma unroll
  for (int s = 0; s < PD; ++s)
#pragma unroll
    for (int j = 0; j < NB; ++j) bq[s][j] = load_bfrag<W4>(b_src[j], e_src[j], min(s, KT - 1));
#pragma unroll
  for (int i = 0; i < CPT; ++i) a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i]);
  hs_stage = hs_src[0];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    if (CH % NTH == 0 || tid + i * NTH < CH)
      *reinterpret_cast<v4i*>(&lds_a[0][a_dst[i]]) = a_stage[i];
  if (tid < BM) hsl[0][tid] = hs_stage;
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i] + min(1, KT - 1) * kBK);
  hs_stage = hs_src[min(1, KT - 1)];
  __syncthreads();

#pragma unroll (KTC > 0 ? KTC : 1)
  for (int kt0 = 0; kt0 < KT; kt0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int kt = kt0 + s;
      if (kt < KT) {
        const int cur = kt & 1;
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const v8i af = lds_afrag(lds_a[cur] + rbase * kBK, i, lane);
          v4f part[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j)
            part[j] = mfma_w(af, bq[s][j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float hs = hsl[cur][rbase + i * 16 + 4 * (lane >> 4) + q];
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j][q] = fmaf(part[j][q], hs, acc[i][j][q]);
          }
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          if (CH % NTH == 0 || tid + i * NTH < CH)
            *reinterpret_cast<v4i*>(&lds_a[cur ^ 1][a_dst[i]]) = a_stage[i];
        if (tid < BM) hsl[cur ^ 1][tid] = hs_stage;
        const int ka = min(kt + 2, KT - 1), kb = min(kt + PD, KT - 1);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
          a_stage[i] = *reinterpret_cast<const v4i*>(a_src[i] + ka * kBK);
        hs_stage = hs_src[ka];
        if constexpr (PAIR) {
          if (s % 2 == 1) {
            const int kb0 = min(kt + PD - 1, KT - 1);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              bq[s - 1][j] = load_bfrag<W4>(b_src[j], e_src[j], kb0);
              bq[s][j] = load_bfrag<W4>(b_src[j], e_src[j], kb);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j) bq[s][j] = load_bfrag<W4>(b_src[j], e_src[j], kb);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: channel scale, bf16 ----
  uint16_t* out = static_cast<uint16_t*>(S.out);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (mcol[j] >= d) continue;
    const float sc = s2v[j];
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rbase + i * 16 + 4 * (lane >> 4) + q;
        if (r < te.nrows)
          out[(size_t)(te.row0 + r) * d + mcol[j]] = f32_to_bf16(acc[i][j][q] * sc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down GEMM for tall tiles (prefill): LDS-staged like the gate/up kernel
// above, with all eight waves in one phase. Tile BM rows x 256 output channels, 8 waves, wave (wm, wn)
// owns rows [wm BM/2, (wm + 1) BM/2) and channels [64 wn, 64 wn + 64). h rows
// (2 stages) and W2 rows (3 stages) arrive by direct loads; a workgroup runs
// NTW consecutive N tiles as one continuous sequence of NTW x KT steps, so
// each group's weights are fetched once and the ring fills once. The per-row
// h block scale of each K step multiplies that step's MFMA partial.
// ---------------------------------------------------------------------------
template <int BM, int KTC, int NTW, bool W4>
__global__ __launch_bounds__(8 * kWave) void down_fp8_lds_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NW = 8, NTH = NW * kWave;
  constexpr int BMW = BM / 2, MS = BMW / 16;
  constexpr int NB = 4;
  constexpr int KB = kstep_bytes<W4>();               // weight bytes per row and K step
  constexpr int NAD = BM * kBK / 1024 / NW;           // A loads per thread per step
  constexpr int NBD = kDownBN * KB / 1024 / NW;       // B loads per thread per step
  constexpr int NSTEP = NTW * KTC;
  constexpr int HCH = BM * KTC / kWave;  // 64-value chunks of the h block scales
  // ... of the channel scales (FP8) or of the MXFP4 scale tile
  constexpr int SCH = W4 ? (NTW * kDownBN * (KTC + 1) + kWave - 1) / kWave : NTW * kDownBN / kWave;
  static_assert(BM * kBK % (1024 * NW) == 0, "A tile must split into whole wave loads");
  static_assert(HCH % NW == 0, "h scale chunks split evenly over the waves");
  static_assert(W4 || SCH <= NW, "one channel-scale chunk per wave at most");

  __shared__ __attribute__((aligned(1024))) uint8_t a0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[kDownBN * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[kDownBN * KB];
  __shared__ __attribute__((aligned(1024))) uint8_t b2[kDownBN * KB];
  // MXFP4 scale tile (whole 64-dword chunks: it is filled by them)
  __shared__ int ssc[W4 ? SCH * kWave : 1];
  __shared__ float hsl[KTC][BM];
  __shared__ __attribute__((aligned(16))) float s2l[W4 ? 1 : NTW * kDownBN];  // channel scales

  const int d = c.d, dnt = down_ntiles(d);
  Tile te;
  if (!pick_tile<BM>(list, hdr->n_down, ceil_div(dnt, NTW), te)) return;
  const int nt0 = te.ntile * NTW;
  const int sid = te.gid >> 16, g = te.gid & 0xffff;
  const SetView S = set_view(c, sid);
  const int F = S.F;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // the wave index in a scalar register frees vector registers on the FP8
  // path (spill-free at 192 rows x 2 N tiles); the MXFP4 path allocates best
  // with it in a vector register
  const int wave = W4 ? tid / kWave : __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / kNWaves, wn = wave % kNWaves;
  const int rbase = wm * BMW;

  // direct-load sources: A load i covers tile rows 8 (NAD wave + i) + lane / 8
  // (a uniform tile base and 32-bit per-lane offsets: fewer vector registers)
  const uint8_t* hbase = S.h + (size_t)te.row0 * F;
  uint32_t aoff[NAD];
#pragma unroll
  for (int i = 0; i < NAD; ++i) {
    const int r = 8 * (NAD * wave + i) + (lane >> 3);
    const int cch = (lane & 7) ^ (r & 7);
    aoff[i] = (uint32_t)min(r, te.nrows - 1) * (uint32_t)F + cch * 16;
  }
  // B load i covers channel rows 8 (NBD wave + i) + lane / 8 of an N tile
  // (MXFP4: 16 rows of 64 bytes, chunk q of row r stored at q ^ ((r / 2) % 4),
  // as in the gate/up kernel); steps past the last N tile re-read its rows
  // (never used)
  const size_t wrb = W4 ? F / 2 : F;
  const uint8_t* w2 = S.w2 + (size_t)g * d * wrb;
  // B piece i of this thread: row brow0 + RPB i of the N tile; its chunk
  // (the swizzle) is the same for every i, since RPB is a multiple of the
  // swizzle period
  constexpr int RPB = W4 ? 16 : 8;  // rows per 1 KiB block
  const int brow0 = RPB * NBD * wave + (W4 ? (lane >> 2) : (lane >> 3));
  const int bcc = W4 ? ((lane & 3) ^ ((brow0 >> 1) & 3)) * 16 : ((lane & 7) ^ (brow0 & 7)) * 16;
  auto load_a = [&](int st, uint8_t* dst) {
    const int kt = st % KTC;
#pragma unroll
    for (int i = 0; i < NAD; ++i) dma16(hbase + aoff[i] + kt * kBK, dst + (NAD * wave + i) * 1024);
  };
  auto load_b = [&](int st, uint8_t* dst) {
    const int n = min(st / KTC, dnt - 1 - nt0), kt = st % KTC;
#pragma unroll
    for (int i = 0; i < NBD; ++i) {
      const int ch = min((nt0 + n) * kDownBN + brow0 + RPB * i, d - 1);
      dma16(w2 + (size_t)ch * wrb + kt * KB + bcc, dst + (NBD * wave + i) * 1024);
    }
  };
  // Prologue: the operands of the first step, every scale the tile needs (h
  // block scales of its rows, every N tile's channel scales or MXFP4 scale
  // rows), then the weights of the second step, all by direct-to-LDS loads
  // issued at once (the first step's wait leaves only the last in flight), so they
  // arrive together (through registers, the scales' LDS writes would wait
  // for their loads before the operands' loads could issue). Scales go in
  // 64-value chunks, one value per lane. (The MFMAs take the weights as A,
  // so lane l accumulates channels 16 j + 4 (l / 16) + q of the wave's 64
  // for tile row 16 i + l % 16.)
  load_b(0, b0);
  load_a(0, a0);
#pragma unroll
  for (int q = 0; q < HCH / NW; ++q) {  // hsl[kt][r] = h_scale[row r][kt]
    const int ci = wave + q * NW, f = ci * kWave + lane;
    const int kt = f / BM, r = f % BM;
    dma4(S.h_scale + (size_t)(te.row0 + min(r, te.nrows - 1)) * KTC + kt, &hsl[0][0] + ci * kWave);
  }
  if constexpr (!W4) {
    if (wave < SCH) {  // s2l[e]: channel (nt0 + e / 256) 256 + e % 256
      const int e = wave * kWave + lane;
      dma4(S.s2 + (size_t)g * d + min((nt0 + e / kDownBN) * kDownBN + e % kDownBN, d - 1),
           s2l + wave * kWave);
    }
  } else {
#pragma unroll
    for (int q = 0; q < (SCH + NW - 1) / NW; ++q) {
      // MXFP4 tile dword r (KTC + 1) + kt: K step kt's four E8M0 scales of
      // tile row r = channel (nt0 + r / 256) 256 + r % 256 (kt = KTC: the
      // row's padding, loaded with a repeated dword)
      const int ci = wave + q * NW, f = ci * kWave + lane;
      if (SCH % NW == 0 || ci < SCH) {
        const int r = min(f / (KTC + 1), NTW * kDownBN - 1), kt = min(f % (KTC + 1), KTC - 1);
        const int n = min(r / kDownBN, dnt - 1 - nt0);
        const int ch = min((nt0 + n) * kDownBN + r % kDownBN, d - 1);
        dma4(reinterpret_cast<const int*>(S.e2 + ((size_t)g * d + ch) * (F / 32) + 4 * kt),
             ssc + ci * kWave);
      }
    }
  }
  if (NSTEP > 1) load_b(1, b1);

  // output rows of this tile, written with buffer stores (masked lanes are
  // dropped by the range check, so each store is one instruction for vmcnt)
  constexpr int NSTV = MS * NB / 2;  // stores per wave per N tile
  const __amdgpu_buffer_rsrc_t orsrc = buffer_rsrc(
      static_cast<uint16_t*>(S.out) + (size_t)te.row0 * d, te.nrows * d * 2);
  v4f acc[MS][NB];
#pragma unroll (NSTEP)
  for (int st = 0; st < NSTEP; ++st) {
    const int kt = st % KTC, n = st / KTC;
    if (kt == 0) {
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // the previous N tile's stores, issued after this step's loads, may
    // stay in flight
    if (st + 1 == NSTEP)
      wait_vmcnt<0>();
    else if (kt == 0 && st > 0)
      wait_vmcnt<NBD + NSTV>();
    else
      wait_vmcnt<NBD>();
    __builtin_amdgcn_s_barrier();  // also publishes hsl on the first step
    uint8_t* as = (st % 2 == 0) ? a0 : a1;
    uint8_t* bs = (st % 3 == 0) ? b0 : (st % 3 == 1) ? b1 : b2;
    if (st + 1 < NSTEP) load_a(st + 1, (st % 2 == 0) ? a1 : a0);
    if (st + 2 < NSTEP) load_b(st + 2, (st % 3 == 0) ? b2 : (st % 3 == 1) ? b0 : b1);
    BFrag<W4> bf[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (W4) {
        const int r = wn * 64 + j * 16 + (lane & 15);
        bf[j].w = *reinterpret_cast<const v4i*>(bs + r * KB + (((lane >> 4) ^ ((r >> 1) & 3)) << 4));
        bf[j].s = scale_from_tile<KTC>(ssc, n * kDownBN + r, kt, lane);
      } else {
        bf[j] = lds_afrag(bs + (wn * 64 + j * 16) * kBK, 0, lane);
      }
    }
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const v8i af = lds_afrag(as + rbase * kBK, i, lane);
      v4f part[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) part[j] = mfma_wt(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f});
      const float hs = hsl[kt][rbase + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(part[j][q], hs, acc[i][j][q]);
    }
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
    if (kt == KTC - 1 && nt0 + n < dnt) {  // this N tile is done: channel scale, bf16
      // Lane l holds 4 channels of subtile j for its row; lanes l and l ^ 16
      // (the same row, neighbouring channel quads) swap one subtile's quad of
      // a pair (j0, j0 + 1), so each lane stores 8 consecutive channels: even
      // lane groups those of j0, odd ones those of j0 + 1. A store then
      // writes 16 rows x 64 contiguous bytes (instead of 32).
      const bool ev = ((lane >> 4) & 1) == 0;
#pragma unroll
      for (int j0 = 0; j0 < NB; j0 += 2) {
        v4f sc0 = v4f{1.f, 1.f, 1.f, 1.f}, sc1 = sc0;
        if constexpr (!W4) {
          const float* sp = &s2l[n * kDownBN + wn * (NB * 16) + j0 * 16 + 4 * (lane >> 4)];
          sc0 = *reinterpret_cast<const v4f*>(sp);
          sc1 = *reinterpret_cast<const v4f*>(sp + 16);
        }
        // channel of the lane's first stored element: 16 (j0 or j0 + 1) +
        // 8 (lane group / 2) of the wave's 64 in N tile n
        const int m = (nt0 + n) * kDownBN + wn * (NB * 16) + (j0 + (ev ? 0 : 1)) * 16 +
                      8 * (lane >> 5);  // d is a multiple of 128: all eight or none
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const v4f a0v = acc[i][j0], a1v = acc[i][j0 + 1];
          const uint32_t p00 = pack_bf16x2(a0v[0] * sc0[0], a0v[1] * sc0[1]);
          const uint32_t p01 = pack_bf16x2(a0v[2] * sc0[2], a0v[3] * sc0[3]);
          const uint32_t p10 = pack_bf16x2(a1v[0] * sc1[0], a1v[1] * sc1[1]);
          const uint32_t p11 = pack_bf16x2(a1v[2] * sc1[2], a1v[3] * sc1[3]);
          // the quad the partner lane stores goes to it, the partner's quad
          // this lane stores comes back: lane l ^ 16 by ds_swizzle in bitmask
          // mode (and 0x1f, or 0, xor 0x10 within each 32 lanes; no address
          // register, unlike a bpermute)
          const uint32_t g0 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(ev ? p10 : p00), 0x401F);
          const uint32_t g1 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(ev ? p11 : p01), 0x401F);
          const __attribute__((ext_vector_type(4))) uint32_t v =
              ev ? (__attribute__((ext_vector_type(4))) uint32_t){p00, p01, g0, g1}
                 : (__attribute__((ext_vector_type(4))) uint32_t){g0, g1, p10, p11};
          const int r = rbase + i * 16 + (lane & 15);
          const int off = (r < te.nrows && m < d) ? (r * d + m) * 2 : -1;
          __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Down GEMM with the tile's h slab resident in LDS (BM x KT x 128 bytes, at
// most 64 KiB: BM <= 64 at F = 1024). The slab and its block scales are
// loaded once; then the workgroup streams the weights of NTW consecutive N
// tiles (256 output channels each) through one continuous K loop of NTW x KT
// steps: each wave keeps PD steps of its weight rows in flight in registers,
// across N-tile boundaries, so the pipeline fills once per workgroup, and
// the K loop has no barrier. With NW waves, wave w owns channels
// [w 256/NW, (w + 1) 256/NW) of every N tile, over all BM rows.
// ---------------------------------------------------------------------------
template <int BM, int KTC, int NTW, int NW, bool W4>
__global__ __launch_bounds__(NW * kWave) void down_fp8_resident_kernel(
    FfnCall c, const TileHeader* __restrict__ hdr, const TileEntry* __restrict__ list) {
  constexpr int NTH = NW * kWave;
  constexpr int MS = BM / 16;
  constexpr int NB = kDownBN / 16 / NW;  // 16-channel subtiles per wave
  constexpr int CHK = BM * (kBK / 16);  // 16-byte chunks per K step
  constexpr int CPT = (CHK * KTC + NTH - 1) / NTH;
  constexpr int GRP = 8;                 // slab chunks per thread per load group
  constexpr int NSTEP = NTW * KTC;
  constexpr int PDM = W4 ? 6 : 4;  // MXFP4: half the bytes per step, deeper ring
  constexpr int PD = NSTEP < PDM ? NSTEP : PDM;
  constexpr bool QS = W4 && KTC % 4 == 0;  // MXFP4 scales held per row for every N tile
  constexpr int KTS = QS ? KTC : 4;
  constexpr bool PAIR = W4 && PD % 2 == 0;   // both halves of a row's line together
  constexpr int HPT = (BM * KTC + NTH - 1) / NTH;
  static_assert(BM * KTC * kBK <= 65536, "h slab exceeds the LDS budget");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[KTC][BM * kBK];
  __shared__ float hsl[KTC][BM];

  const int d = c.d, dnt = down_ntiles(d);
  Tile te;
  if (!pick_tile<BM>(list, hdr->n_down, ceil_div(dnt, NTW), te)) return;
  const int nt0 = te.ntile * NTW;
  const int sid = te.gid >> 16, g = te.gid & 0xffff;
  const SetView S = set_view(c, sid);
  const int F = S.F;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wn = tid / kWave;

  const size_t wrb = W4 ? F / 2 : F;  // weight bytes per row
  const uint8_t* w2 = S.w2 + (size_t)g * d * wrb + (lane >> 4) * 16;
  const uint8_t* e2 = W4 ? S.e2 + (size_t)g * d * (F / 32) + (lane >> 4) : nullptr;
  // output channel of (N tile n of this workgroup, subtile j) for this lane
  auto mcol = [&](int n, int j) {
    return (nt0 + n) * kDownBN + wn * (NB * 16) + j * 16 + (lane & 15);
  };
  // weight fragment of step s (N tile s / KT, K step s % KT); steps past the
  // last N tile re-read its rows (never used)
  auto bfrag = [&](int st, int j) {
    const int n = min(st / KTC, dnt - 1 - nt0);
    const size_t row = min(mcol(n, j), d - 1);
    return load_bfrag<W4, !QS>(w2 + row * wrb, W4 ? e2 + row * (F / 32) : nullptr, st % KTC);
  };
  // MXFP4 scales of every N tile's rows (QS)
  int srow[NTW][NB][KTS / 4];
  if constexpr (QS) {
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int nn = min(n, dnt - 1 - nt0);
        load_scale_row<KTS>(srow[n][j], S.e2 + ((size_t)g * d + min(mcol(nn, j), d - 1)) * (F / 32),
                            lane);
      }
  }
  // channel scales of every N tile, loaded now so the epilogues wait on no load
  float s2v[NTW][NB];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      s2v[n][j] = W4 ? 1.f : S.s2[(size_t)g * d + min(mcol(n, j), d - 1)];
  float hv[HPT];
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int e = min(tid + i * NTH, BM * KTC - 1);
    const int r = e / KTC, kt = e % KTC;
    hv[i] = S.h_scale[(size_t)(te.row0 + min(r, te.nrows - 1)) * KTC + kt];
  }
  // The h slab in groups of GRP chunks per thread (chunk ch = (step, row,
  // 16-byte column); rows past the tile's end repeat its last row and are
  // never stored). The weight ring is issued after the first group, so the
  // first group's stores wait for that group alone.
  BFrag<W4> bq[PD][NB];
#pragma unroll
  for (int g0 = 0; g0 < CPT; g0 += GRP) {
    v4i st[GRP];
    int dst[GRP];
#pragma unroll
    for (int i = 0; i < GRP; ++i) {
      if (g0 + i < CPT) {
        const int ch = min(tid + (g0 + i) * NTH, CHK * KTC - 1);
        const int kt = ch / CHK, cc = ch % CHK;
        const int r = cc >> 3, c16 = cc & 7;
        const size_t grow = (size_t)(te.row0 + min(r, te.nrows - 1));
        st[i] = *reinterpret_cast<const v4i*>(S.h + grow * F + kt * kBK + c16 * 16);
        dst[i] = kt * (BM * kBK) + swz(r, c16);
      }
    }
    if (g0 == 0) {
#pragma unroll
      for (int s = 0; s < PD; ++s)
#pragma unroll
        for (int j = 0; j < NB; ++j) bq[s][j] = bfrag(s, j);
    }
#pragma unroll
    for (int i = 0; i < GRP; ++i)
      if (g0 + i < CPT && ((CHK * KTC) % NTH == 0 || tid + (g0 + i) * NTH < CHK * KTC))
        *reinterpret_cast<v4i*>(&lds_a[0][0] + dst[i]) = st[i];
  }
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int e = tid + i * NTH;
    if ((BM * KTC) % NTH == 0 || e < BM * KTC) hsl[e % KTC][e / KTC] = hv[i];
  }
  __syncthreads();

  uint16_t* out = static_cast<uint16_t*>(S.out);
  v4f acc[MS][NB];
#pragma unroll (NSTEP)
  for (int st = 0; st < NSTEP; ++st) {
    const int s = st % PD, kt = st % KTC, n = st / KTC;
    if (kt == 0) {
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (QS) {
#pragma unroll
      for (int j = 0; j < NB; ++j) bq[s][j].s = scale_of_step<KTS>(srow[n][j], kt, lane);
    }
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const v8i af = lds_afrag(lds_a[kt], i, lane);
      v4f part[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        part[j] = mfma_w(af, bq[s][j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float hs = hsl[kt][i * 16 + 4 * (lane >> 4) + q];
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j][q] = fmaf(part[j][q], hs, acc[i][j][q]);
      }
    }
    if constexpr (PAIR) {
      if (st % 2 == 1) {  // PD even: slot s - 1 held step st - 1
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (st + PD - 1 < NSTEP) bq[s - 1][j] = bfrag(st + PD - 1, j);
          if (st + PD < NSTEP) bq[s][j] = bfrag(st + PD, j);
        }
      }
    } else if (st + PD < NSTEP) {
#pragma unroll
      for (int j = 0; j < NB; ++j) bq[s][j] = bfrag(st + PD, j);
    }

    // keep each step's loads and scaled accumulation in the step (the
    // scheduler would otherwise sink the loads towards their use, shortening
    // the ring, and hold every partial product live to the end)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
    if (kt == KTC - 1 && nt0 + n < dnt) {  // this N tile is done: channel scale, bf16
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int m = mcol(n, j);
        if (m >= d) continue;
#pragma unroll
        for (int i = 0; i < MS; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = i * 16 + 4 * (lane >> 4) + q;
            if (r < te.nrows)
              out[(size_t)(te.row0 + r) * d + m] = f32_to_bf16(acc[i][j][q] * s2v[n][j]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// float32 path: one thread per output element, plain sequential dot products.
// ---------------------------------------------------------------------------
__device__ inline int find_group(const FfnSet& S, int r) {
  if (S.offsets == nullptr) return (r < min(S.rows_fixed, S.max_rows)) ? 0 : -1;
  if (r >= S.offsets[S.G]) return -1;
  int a = 0, b = S.G;  // offsets[a] <= r < offsets[b]
  while (b - a > 1) {
    const int m = (a + b) >> 1;
    if (S.offsets[m] <= r) a = m; else b = m;
  }
  return a;
}

__global__ __launch_bounds__(256) void gateup_f32_kernel(FfnCall c, int sid) {
  const FfnSet S = (sid == 0) ? c.set[0] : c.set[1];
  const int F = S.F, d = c.d;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)S.max_rows * F) return;
  const int r = (int)(idx / F), n = (int)(idx % F);
  const int g = find_group(S, r);
  if (g < 0) return;
  const int src = min(max(S.row_src ? S.row_src[r] / S.src_div : r, 0), c.a_rows - 1);
  const float* x = static_cast<const float*>(c.a) + (size_t)src * d;
  const float* w = reinterpret_cast<const float*>(S.w13) + (size_t)g * 2 * F * d;
  const float* wg = w + (size_t)n * d;
  const float* wu = w + (size_t)(F + n) * d;
  float gv = 0.f, uv = 0.f;
  for (int i = 0; i < d; ++i) {
    gv = fmaf(x[i], wg[i], gv);
    uv = fmaf(x[i], wu[i], uv);
  }
  reinterpret_cast<float*>(S.h)[(size_t)r * F + n] = gv / (1.0f + expf(-gv)) * uv;
}

__global__ __launch_bounds__(256) void down_f32_kernel(FfnCall c, int sid) {
  const FfnSet S = (sid == 0) ? c.set[0] : c.set[1];
  const int F = S.F, d = c.d;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)S.max_rows * d) return;
  const int r = (int)(idx / d), m = (int)(idx % d);
  const int g = find_group(S, r);
  if (g < 0) return;
  const float* h = reinterpret_cast<const float*>(S.h) + (size_t)r * F;
  const float* w = reinterpret_cast<const float*>(S.w2) + (size_t)g * d * F + (size_t)m * F;
  float acc = 0.f;
  for (int n = 0; n < F; ++n) acc = fmaf(h[n], w[n], acc);
  static_cast<float*>(S.out)[(size_t)r * d + m] = acc;
}

// Compute units of the current device, looked up once per device (the
// persistent gate/up kernel runs one workgroup per compute unit).
hipError_t device_cus(int* out) {
  static std::atomic<int> cus[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return hipSuccess;
}

// Waves along M for a tile height: one for decode-sized tiles, two from 64 rows.
template <int BM>
constexpr int waves_m() { return BM >= 64 ? 2 : 1; }

// W4: MXFP4 weights (every kernel has an MXFP4 variant).
template <int BM, int KTU, int BMD, int KTD, bool W4>
hipError_t launch_gemms_bm(const FfnCall& c, TileHeader* hdr, TileEntry* up, TileEntry* dn,
                           size_t cap_u, size_t cap_d, hipStream_t s, const StepEvents& ev) {
  const size_t cu = align_up(cap_u * up_ntiles_max(c), kXcds);
  const size_t cd = align_up(cap_d * down_ntiles(c.d), kXcds);
  constexpr int WU = waves_m<BM>(), WD = waves_m<BMD>();
  ev.mark(true, MOE_STEP_GATE_UP, s);
  if (cu > 0) {
    if constexpr (KTU > 0 && BM == 192) {
      // tallest tiles: one wave per SIMD, one workgroup per compute unit
      // (a multiple of the XCD count, as the tile order assumes), each
      // working through its XCD's tiles
      int ncu = 0;
      const hipError_t e = device_cus(&ncu);
      if (e != hipSuccess) return e;
      const size_t grid = std::min(cu, (size_t)std::max(kXcds, ncu / kXcds * kXcds));
      hipLaunchKernelGGL((gateup_fp8_iw_kernel<BM, KTU, W4>), dim3((unsigned)grid),
                         dim3(4 * kWave), 0, s, c, hdr, up);
    }
    else if constexpr (KTU > 0 && BM >= 128)  // tall tiles: ping-pong schedule
      hipLaunchKernelGGL((gateup_fp8_pp_kernel<BM, KTU, pp_weight_stages<BM, W4>(), W4>),
                         dim3((unsigned)cu), dim3(8 * kWave), 0, s, c, hdr, up);
    else  // (a fully unrolled K loop of tall tiles would spill: looped there)
      hipLaunchKernelGGL((gateup_fp8_kernel<BM, WU, (BM >= 128 ? 0 : KTU), W4>),
                         dim3((unsigned)cu), dim3(kNWaves * WU * kWave), 0, s, c, hdr, up);
  }
  ev.mark(false, MOE_STEP_GATE_UP, s);
  ev.mark(true, MOE_STEP_DOWN, s);
  if (cap_d > 0) {
    if constexpr (KTD > 0 && BMD >= 128) {
      // tall tiles: both operands through LDS, 16 steps per workgroup
      constexpr int NTW = KTD >= 16 ? 1 : 16 / KTD;
      const size_t cdl = align_up(cap_d * ceil_div(down_ntiles(c.d), NTW), kXcds);
      hipLaunchKernelGGL((down_fp8_lds_kernel<BMD, KTD, NTW, W4>), dim3((unsigned)cdl),
                         dim3(8 * kWave), 0, s, c, hdr, dn);
    } else if constexpr (KTD > 0 && BMD * KTD * kBK <= 65536) {
      // resident h slab; 64-row tiles: 8 waves, 4 N tiles per workgroup;
      // MXFP4 weights (half the bytes per K step) also take 8 waves at 16
      // and 32 rows, so a workgroup keeps as many weight bytes in flight
      // (FP8 measured slower at 8: 97 against 94 us at decode, MXFP4 faster:
      // 53 against 55)
      constexpr int NTW = BMD >= 64 ? 4 : 1, NWD = (BMD >= 64 || W4) ? 8 : 4;
      const size_t cdr = align_up(cap_d * ceil_div(down_ntiles(c.d), NTW), kXcds);
      hipLaunchKernelGGL((down_fp8_resident_kernel<BMD, KTD, NTW, NWD, W4>), dim3((unsigned)cdr),
                         dim3(NWD * kWave), 0, s, c, hdr, dn);
    } else {
      hipLaunchKernelGGL((down_fp8_kernel<BMD, WD, KTD, W4>), dim3((unsigned)cd),
                         dim3(kNWaves * WD * kWave), 0, s, c, hdr, dn);
    }
  }
  ev.mark(false, MOE_STEP_DOWN, s);
  return hipGetLastError();
}

// The K loops are fully unrolled where the compile-time step counts match
// the call: 32 gate/up steps (d = 4096); 8 down steps (F = 1024, every set)
// for the resident and the tall-tile down kernels, or 16 (F = 2048) for the
// tall-tile one. Other sizes use the looped kernels.
template <int BM, int BMD, int KTU, bool W4>
hipError_t launch_gemms_kd(const FfnCall& c, TileHeader* hdr, TileEntry* up, TileEntry* dn,
                           size_t cap_u, size_t cap_d, hipStream_t s, const StepEvents& ev) {
  const int kdn = down_ksteps(c);
  if constexpr (BMD <= 64 || BMD >= 128) {
    if (kdn == 8)
      return launch_gemms_bm<BM, KTU, BMD, 8, W4>(c, hdr, up, dn, cap_u, cap_d, s, ev);
  }
  if constexpr (BMD >= 128) {
    if (kdn == 16)
      return launch_gemms_bm<BM, KTU, BMD, 16, W4>(c, hdr, up, dn, cap_u, cap_d, s, ev);
  }
  if constexpr (BMD <= 128)  // taller down tiles exist only where K is fixed (above)
    return launch_gemms_bm<BM, KTU, BMD, 0, W4>(c, hdr, up, dn, cap_u, cap_d, s, ev);
  return hipErrorInvalidValue;
}

template <int BM, int BMD, bool W4>
hipError_t launch_gemms_k(const FfnCall& c, TileHeader* hdr, TileEntry* up, TileEntry* dn,
                          size_t cap_u, size_t cap_d, hipStream_t s, const StepEvents& ev) {
  if (c.d / kBK == 32)
    return launch_gemms_kd<BM, BMD, 32, W4>(c, hdr, up, dn, cap_u, cap_d, s, ev);
  return launch_gemms_kd<BM, BMD, 0, W4>(c, hdr, up, dn, cap_u, cap_d, s, ev);
}

template <bool W4>
hipError_t launch_gemms_w(const FfnCall& c, int bm, TileHeader* hdr, TileEntry* up,
                          TileEntry* dn, int cu, int cd, hipStream_t s, const StepEvents& ev) {
  switch (bm) {
    case 16: return launch_gemms_k<16, 16, W4>(c, hdr, up, dn, cu, cd, s, ev);
    case 32: return launch_gemms_k<32, 32, W4>(c, hdr, up, dn, cu, cd, s, ev);
    case 64: return launch_gemms_k<64, 64, W4>(c, hdr, up, dn, cu, cd, s, ev);
    case 128: return launch_gemms_k<128, 128, W4>(c, hdr, up, dn, cu, cd, s, ev);
    default:
      return down_bm(c, bm) == 192 ? launch_gemms_k<192, 192, W4>(c, hdr, up, dn, cu, cd, s, ev)
                                   : launch_gemms_k<192, 128, W4>(c, hdr, up, dn, cu, cd, s, ev);
  }
}

}  // namespace

size_t ffn_tiles_ws_bytes(const FfnCall& c) {
  // capacity for the smallest tile height (the largest list)
  return align_up(sizeof(TileHeader) + 2 * tiles_cap(c, 16) * sizeof(TileEntry), 256);
}

size_t ffn_h_bytes(int max_rows, int F, bool fp8) {
  return align_up((size_t)max_rows * F * (fp8 ? 1 : sizeof(float)), 256);
}

size_t ffn_hs_bytes(int max_rows, int F) {
  return align_up((size_t)max_rows * (F / kHN) * sizeof(float), 256);
}

int choose_bm(int rows_hint) {
  // fewest (M tiles x (BM + 64)): 64 rows' worth of cost per tile for
  // streaming its weights, BM rows of MFMA work (padding included)
  static const int cand[] = {16, 32, 64, 128, 192};
  int best = 16;
  long best_cost = -1;
  for (int bm : cand) {
    const long cost = (long)ceil_div(max(rows_hint, 1), bm) * (bm + 64);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = bm;
    }
  }
  return best;
}

void tile_lists(const FfnCall& c, int bm, void* ws, TileHeader** hdr, TileEntry** up,
                TileEntry** dn, int* cap_up, int* cap_dn) {
  *hdr = static_cast<TileHeader*>(ws);
  *up = reinterpret_cast<TileEntry*>(*hdr + 1);
  *dn = *up + tiles_cap(c, 16);
  *cap_up = (int)tiles_cap(c, bm);
  *cap_dn = (int)tiles_cap(c, down_bm(c, bm));
}

hipError_t launch_ffn_tiles(const FfnCall& c, int bm, void* ws, hipStream_t s) {
  TileHeader* hdr;
  TileEntry *up, *dn;
  int cu, cd;
  tile_lists(c, bm, ws, &hdr, &up, &dn, &cu, &cd);
  hipLaunchKernelGGL(ffn_tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, c, bm, hdr, up, dn, cu, cd);
  return hipGetLastError();
}

hipError_t launch_ffn_gemms(const FfnCall& c, int bm, void* ws, hipStream_t s,
                            const StepEvents& ev) {
  TileHeader* hdr;
  TileEntry *up, *dn;
  int cu, cd;
  tile_lists(c, bm, ws, &hdr, &up, &dn, &cu, &cd);
  if (c.set[0].w4) return launch_gemms_w<true>(c, bm, hdr, up, dn, cu, cd, s, ev);
  return launch_gemms_w<false>(c, bm, hdr, up, dn, cu, cd, s, ev);
}

hipError_t launch_grouped_ffn_fp8(const FfnCall& c, void* tiles_ws, int rows_hint, hipStream_t s,
                                  const StepEvents& ev) {
  const int bm = choose_bm(rows_hint);
  ev.mark(true, MOE_STEP_TILES, s);
  hipError_t e = launch_ffn_tiles(c, bm, tiles_ws, s);
  ev.mark(false, MOE_STEP_TILES, s);
  if (e != hipSuccess) return e;
  return launch_ffn_gemms(c, bm, tiles_ws, s, ev);
}

hipError_t launch_grouped_ffn_f32(const FfnCall& c, hipStream_t s, const StepEvents& ev) {
  ev.mark(true, MOE_STEP_GATE_UP, s);
  for (int sid = 0; sid < c.nsets; ++sid) {
    const FfnSet& S = c.set[sid];
    const size_t nu = (size_t)S.max_rows * S.F;
    if (nu > 0)
      hipLaunchKernelGGL(gateup_f32_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, s, c, sid);
  }
  ev.mark(false, MOE_STEP_GATE_UP, s);
  ev.mark(true, MOE_STEP_DOWN, s);
  for (int sid = 0; sid < c.nsets; ++sid) {
    const FfnSet& S = c.set[sid];
    const size_t nd = (size_t)S.max_rows * c.d;
    if (nd > 0)
      hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, s, c, sid);
  }
  ev.mark(false, MOE_STEP_DOWN, s);
  return hipGetLastError();
}

}  // namespace moe
