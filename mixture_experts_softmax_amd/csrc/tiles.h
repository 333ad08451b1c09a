// Grouped-FFN work lists: for every non-empty group, one entry per M tile (up
// to BM rows each), one list for the gate/up GEMM (tile height bm) and one
// for the down GEMM (down_bm(c, bm)). A GEMM launch covers (list entry, N tile)
// pairs; the block index selects the pair. Emitted by one workgroup; used by
// the tile-list kernel of moe_grouped_ffn and by the permutation of
// moe_layer_forward (which knows the group sizes first).
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kHN = 128;      // h columns per gate/up tile = one h quantisation block
constexpr int kDownBN = 256;  // output channels per down tile
constexpr int kMaxGroups = 1024;

// One entry per M tile of a group; every entry of a group holds the group's
// data (a block finds its M tile from the entry's position).
struct TileEntry {
  int row0;   // first row of the group, in the set's grouped row space
  int rows;   // rows of the group (> 0)
  int gid;    // (set << 16) | group
  int first;  // index of the group's first entry in this list
};

struct TileHeader {
  int n_up;    // entries in the gate/up list
  int n_down;  // entries in the down list
  int pad[62];
};

__host__ __device__ inline int up_ntiles(int F) { return F / kHN; }
__host__ __device__ inline int down_ntiles(int d) { return ceil_div(d, kDownBN); }
// N tiles of a gate/up launch: the widest set's h blocks (blocks past a
// narrower set's width exit at once).
__host__ __device__ inline int up_ntiles_max(const FfnCall& c) {
  const int f = (c.nsets > 1 && c.set[1].F > c.set[0].F) ? c.set[1].F : c.set[0].F;
  return up_ntiles(f);
}

// LDS state of the emitter; the caller fills g_row0/g_rows/g_set for NG groups.
struct TileLds {
  int g_row0[kMaxGroups];
  int g_rows[kMaxGroups];
  int g_set[kMaxGroups];
  int pre_up[kMaxGroups + 1];  // exclusive prefix of the groups' list entries
  int pre_dn[kMaxGroups + 1];
  int wtot_up[16];             // per-wave totals of one scan chunk
  int wtot_dn[16];
};

// Host: where the lists of call c live in its tile workspace, and their
// capacities for gate/up tile height bm (down: down_bm(c, bm)).
void tile_lists(const FfnCall& c, int bm, void* ws, TileHeader** hdr, TileEntry** up,
                TileEntry** dn, int* cap_up, int* cap_dn);

// K steps of the down GEMM when every set has the same F of 1024 or 2048
// (the shapes with fully unrolled down kernels), else 0.
__host__ __device__ inline int down_ksteps(const FfnCall& c) {
  const int f = c.set[0].F;
  if (c.nsets > 1 && c.set[1].F != f) return 0;
  return (f == 1024 || f == 2048) ? f / kHN : 0;
}

// Tile height of the down GEMM for a gate/up tile height: the same up to 32
// rows; 64 rows stay 64 (h slab resident in LDS when F = 1024); taller tiles
// keep their height where the tall-tile kernel's K is fixed (F = 1024 or
// 2048), else at most 128 (the looped kernel's register tile).
__host__ __device__ inline int down_bm(const FfnCall& c, int bm_up) {
  if (bm_up <= 64) return bm_up;
  if (down_ksteps(c) > 0) return bm_up;
  return bm_up < 128 ? bm_up : 128;
}

// All threads of the block (at most 1024) call this after the group arrays are
// filled and synchronised. cap_up / cap_dn bound the lists (entries beyond are
// dropped, which only happens for malformed group offsets).
//   1. M tiles per group, exclusive block-wide scan (chunks of the block
//      size: wave scans, then the wave totals);
//   2. one thread per list entry: its group is the last one whose prefix is
//      not above the entry's index (binary search; empty groups never match).
__device__ inline void emit_tiles(const FfnCall& c, int bm, int NG, int G0, TileLds& L,
                                  TileHeader* hdr, TileEntry* up, TileEntry* down, int cap_up,
                                  int cap_dn) {
  const int bmd = down_bm(c, bm);
  const int tid = threadIdx.x, nth = blockDim.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nth / kWave;
  int carry_u = 0, carry_d = 0;  // identical in every thread
  for (int base = 0; base < NG; base += nth) {
    const int i = base + tid;
    int cu = 0, cd = 0;
    if (i < NG) {
      const int rows = L.g_rows[i];
      cu = ceil_div(rows, bm);
      cd = ceil_div(rows, bmd);
    }
    const int iu = wave_incl_scan(cu, lane), id = wave_incl_scan(cd, lane);
    if (lane == kWave - 1) {
      L.wtot_up[wave] = iu;
      L.wtot_dn[wave] = id;
    }
    __syncthreads();
    int pu = carry_u, pd = carry_d, tu = 0, td = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int a = L.wtot_up[w], b = L.wtot_dn[w];
      if (w < wave) {
        pu += a;
        pd += b;
      }
      tu += a;
      td += b;
    }
    if (i < NG) {
      L.pre_up[i] = pu + iu - cu;
      L.pre_dn[i] = pd + id - cd;
    }
    carry_u += tu;
    carry_d += td;
    __syncthreads();  // wave totals are rewritten by the next chunk
  }
  if (tid == 0) {
    L.pre_up[NG] = carry_u;
    L.pre_dn[NG] = carry_d;
  }
  const int n_up = min(carry_u, cap_up), n_dn = min(carry_d, cap_dn);
  __syncthreads();
  for (int idx = tid; idx < n_up + n_dn; idx += nth) {
    const bool is_up = idx < n_up;
    const int j = is_up ? idx : idx - n_up;
    const int* pre = is_up ? L.pre_up : L.pre_dn;
    int lo = 0, hi = NG - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= j)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int s = L.g_set[lo];
    TileEntry e;
    e.row0 = L.g_row0[lo];
    e.rows = L.g_rows[lo];
    e.gid = (s << 16) | (s == 0 ? lo : lo - G0);
    e.first = pre[lo];
    (is_up ? up : down)[j] = e;
  }
  if (tid == 0) {
    hdr->n_up = n_up;
    hdr->n_down = n_dn;
  }
}

// The same lists written by one wave that holds the routed groups' sizes
// (the fused decode permutation, a few rows per group; with many M tiles per
// group the block-wide emit_tiles is faster):
// lane l holds groups [l PER, (l + 1) PER) of the E routed ones (sizes cnt[],
// the first starting at grouped row row0); the shared expert's group (set 1,
// if present) follows them. The wave scans the groups' M-tile counts and each
// lane writes its own groups' entries, the last lane also the shared group's
// and the header: the entries and positions emit_tiles writes, without its
// block-wide scan or per-entry search.
// Inclusive scan over the 64 lanes by DPP: row shifts by 1, 2, 4 and 8 (zero
// past the row start) scan each row of 16, then the last lane of row 0 is
// added to rows 1 and 3 (row_bcast:15) and that of row 1 to rows 2 and 3
// (row_bcast:31). No LDS round trips, unlike the shuffle scan.
__device__ inline int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// ceil(x / b) for b > 0, by a shift when b is a power of two
__device__ inline int ceil_div_p2(int x, int b) {
  return (b & (b - 1)) == 0 ? (x + b - 1) >> __builtin_ctz(b) : ceil_div(x, b);
}

template <int PER>
__device__ inline void emit_tiles_wave(const FfnCall& c, int bm, int E, const int (&cnt)[PER],
                                       int row0, int lane, TileHeader* hdr, TileEntry* up,
                                       TileEntry* down, int cap_up, int cap_dn) {
  const int bmd = down_bm(c, bm);
  int mu_[PER], md_[PER], su = 0, sd = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    mu_[i] = ceil_div_p2(cnt[i], bm);
    md_[i] = ceil_div_p2(cnt[i], bmd);
    su += mu_[i];
    sd += md_[i];
  }
  int pu = wave_incl_scan_dpp(su) - su, pd = wave_incl_scan_dpp(sd) - sd;
  auto put = [](TileEntry* list, int cap, int first, int n, const TileEntry& te) {
    for (int m = 0; m < n; ++m)
      if (first + m < cap) list[first + m] = te;
  };
  int r0 = row0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * PER + i;
    if (e < E && cnt[i] > 0) {
      const int mu = mu_[i], md = md_[i];
      put(up, cap_up, pu, mu, TileEntry{r0, cnt[i], e, pu});
      put(down, cap_dn, pd, md, TileEntry{r0, cnt[i], e, pd});
      pu += mu;
      pd += md;
    }
    r0 += cnt[i];
  }
  if (lane == kWave - 1) {  // holds the routed totals
    const int nsh = c.nsets > 1 ? min(c.set[1].rows_fixed, c.set[1].max_rows) : 0;
    if (nsh > 0) {
      const int mu = ceil_div_p2(nsh, bm), md = ceil_div_p2(nsh, bmd);
      put(up, cap_up, pu, mu, TileEntry{0, nsh, 1 << 16, pu});
      put(down, cap_dn, pd, md, TileEntry{0, nsh, 1 << 16, pd});
      pu += mu;
      pd += md;
    }
    hdr->n_up = min(pu, cap_up);
    hdr->n_down = min(pd, cap_dn);
  }
}

}  // namespace moe
