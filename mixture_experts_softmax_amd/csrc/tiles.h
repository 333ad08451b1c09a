// Grouped-FFN work lists: for every non-empty group, its M tiles (up to BM
// rows) times its N tiles, the M tiles of one (group, N tile) adjacent so
// that consecutive list entries share weights. Emitted by one workgroup;
// used by the tile-list kernel of moe_grouped_ffn and by the permutation scan
// of moe_layer_forward (which knows the group sizes first).
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kHN = 128;      // h columns per gate/up tile = one h quantisation block
constexpr int kDownBN = 256;  // output channels per down tile
constexpr int kMaxGroups = 1024;

struct TileEntry {
  int row0;   // first row of the tile, in the set's grouped row space
  int nrows;  // rows in this tile, 1..BM
  int gid;    // (set << 16) | group
  int ntile;  // N tile index
};

struct TileHeader {
  int n_up;
  int n_down;
  int pad[62];
};

__host__ __device__ inline int up_ntiles(int F) { return F / kHN; }
__host__ __device__ inline int down_ntiles(int d) { return ceil_div(d, kDownBN); }

// LDS state of the emitter; the caller fills g_row0/g_rows/g_set for NG groups.
struct TileLds {
  int g_row0[kMaxGroups];
  int g_rows[kMaxGroups];
  int g_set[kMaxGroups];
  int pre_up[kMaxGroups + 1];
  int pre_dn[kMaxGroups + 1];
};

// Host: where the lists of call c live in its tile workspace, and their
// capacities for tile height bm.
void tile_lists(const FfnCall& c, int bm_up, int bm_dn, void* ws, TileHeader** hdr,
                TileEntry** up, TileEntry** dn, int* cap_up, int* cap_dn);

// Tile height of the down GEMM for a gate/up tile height (its register tile
// holds no more than 128 rows).
__host__ __device__ inline int down_bm(int bm_up) { return bm_up < 128 ? bm_up : 128; }

// All threads of the block call this after the group arrays are filled and
// synchronised. cap_up / cap_dn bound the lists (entries beyond are dropped,
// which only happens for malformed group offsets).
__device__ inline void emit_tiles(const FfnCall& c, int bm, int NG, int G0, TileLds& L,
                                  TileHeader* hdr, TileEntry* up, TileEntry* down, int cap_up,
                                  int cap_dn) {
  const int bmd = down_bm(bm);
  const int tid = threadIdx.x, nth = blockDim.x;
  const int dnt = down_ntiles(c.d);
  const int F0 = c.set[0].F, F1 = c.set[1].F;
  // exclusive scans of the per-group entry counts, by wave 0 (lane owns a run
  // of groups; a shuffle scan over the lanes)
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nth / kWave;
  if (wave == 0) {
    const int per = ceil_div(NG, kWave);
    const int lo = min(NG, lane * per), hi = min(NG, lo + per);
    int su = 0, sd = 0;
    for (int i = lo; i < hi; ++i) {
      su += ceil_div(L.g_rows[i], bm) * up_ntiles(L.g_set[i] == 0 ? F0 : F1);
      sd += ceil_div(L.g_rows[i], bmd) * dnt;
    }
    const int iu = wave_incl_scan(su, lane), id = wave_incl_scan(sd, lane);
    su = iu - su;
    sd = id - sd;
    for (int i = lo; i < hi; ++i) {
      L.pre_up[i] = su;
      L.pre_dn[i] = sd;
      su += ceil_div(L.g_rows[i], bm) * up_ntiles(L.g_set[i] == 0 ? F0 : F1);
      sd += ceil_div(L.g_rows[i], bmd) * dnt;
    }
    if (lane == kWave - 1) {
      L.pre_up[NG] = iu;
      L.pre_dn[NG] = id;
    }
  }
  __syncthreads();
  // one wave per group writes its entries
  for (int i = wave; i < NG; i += nwaves) {
    const int rows = L.g_rows[i];
    if (rows == 0) continue;
    const int mt = ceil_div(rows, bm), mtd = ceil_div(rows, bmd);
    const int s = L.g_set[i];
    const int gid = (s << 16) | (s == 0 ? i : i - G0);
    const int nu = mt * up_ntiles(s == 0 ? F0 : F1), nd = mtd * dnt;
    for (int j = lane; j < nu + nd; j += kWave) {
      const bool is_up = j < nu;
      const int loc = is_up ? j : j - nu;
      const int idx = (is_up ? L.pre_up[i] : L.pre_dn[i]) + loc;
      if (idx >= (is_up ? cap_up : cap_dn)) continue;
      const int h = is_up ? bm : bmd, m = loc % (is_up ? mt : mtd);
      TileEntry e;
      e.row0 = L.g_row0[i] + m * h;
      e.nrows = min(h, rows - m * h);
      e.gid = gid;
      e.ntile = loc / (is_up ? mt : mtd);
      (is_up ? up : down)[idx] = e;
    }
  }
  if (tid == 0) {
    hdr->n_up = min(L.pre_up[NG], cap_up);
    hdr->n_down = min(L.pre_dn[NG], cap_dn);
  }
}

}  // namespace moe
