// Internal launch interface between the C ABI layer (api.hip) and the kernel
// files. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Tokens per router workgroup and per permutation tile.
constexpr int kRouteTokens = 16;
constexpr int kPermTile = 64;

// ----- router ---------------------------------------------------------------
struct FfnCall;
// Optional fused permutation for a batch of at most kPermTile tokens: the
// top-k workgroup writes offsets, sorted_pair and pair_to_row, and with c and
// tiles_ws also the grouped-FFN tile lists of c for tile height bm.
struct RoutePermute {
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_to_row;
  const FfnCall* c;
  int bm;
  void* tiles_ws;
};
// ws: the K-split partial logits (route_ws_bytes). masks/counts (optional,
// [ceil(T/64)][E]) get the permutation's per-tile expert masks and counts;
// ignored when the permutation is fused (T <= kPermTile and fuse != nullptr).
size_t route_ws_bytes(int T, int d, int E);
// after_logits (optional): recorded on s between the logits launch (which
// writes xq and x_scale) and the selection launch.
hipError_t launch_route(bool bf16, const void* x, const void* w_router, const float* bias, int T,
                        int d, int E, int k, int32_t* ids, float* w, uint8_t* xq, float* x_scale,
                        void* ws, uint64_t* masks, int32_t* counts, const RoutePermute* fuse,
                        hipStream_t s, hipEvent_t after_logits = nullptr);

// ----- permutation ----------------------------------------------------------
size_t perm_masks_bytes(int T, int E);
size_t perm_counts_bytes(int T, int E);
size_t permute_ws_bytes(int T, int E);
// tile_counts (optional): [ceil(T/64)][E] per-tile expert counts.
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_row, int32_t* tile_counts,
                          void* ws, hipStream_t s);
// tile_counts[i] = popcount(masks[i]) over the [ceil(T/64)][E] tile masks.
hipError_t launch_tile_counts(const uint64_t* masks, int T, int E, int32_t* tile_counts,
                              hipStream_t s);
// x_perm[r] = xq[sorted_pair[r] / k] (d bytes) and x_perm_scale[r] = x_scale[...]
// for every row r below offsets[E].
hipError_t launch_perm_gather(const uint8_t* xq, const float* x_scale, const int32_t* sorted_pair,
                              const int32_t* offsets, int T, int E, int k, int d, uint8_t* x_perm,
                              float* x_perm_scale, hipStream_t s);
// x rows to quantise to FP8 (quant.h): T rows of d bf16 values at x, their
// codes to xq [T][d] and scales to xs [T]; T = 0: none.
struct QuantRows {
  const uint16_t* x;
  int T, d;
  uint8_t* xq;
  float* xs;
};
// scan + scatter from masks/counts already computed (counts become the tile
// bases); with c != nullptr also writes the grouped-FFN tile lists of c; with
// quant != nullptr the scan launch also quantises those rows.
hipError_t launch_perm_scan_scatter(const int32_t* ids, int T, int E, int k, uint64_t* masks,
                                    int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                    int32_t* pair_to_row, const FfnCall* c, int bm, void* tiles_ws,
                                    hipStream_t s, const QuantRows* quant = nullptr);

// ----- QK-Norm + RoPE (shape already validated) --------------------------------
hipError_t launch_qk_norm_rope(const moe_qk_shape_t& s, void* qkv, const int32_t* positions,
                               const void* q_weight, const void* k_weight, hipStream_t st);

// ----- grouped FFN ----------------------------------------------------------
// A "set" is a family of groups sharing one weight layout: the routed experts
// (G groups, row ranges from a device offsets array, activation rows gathered
// through row_src) or the shared expert (one group over `rows_fixed` rows).
struct FfnSet {
  const uint8_t* w13;    // [G][2F][d] (bytes: FP8 codes, or float32 when f32);
                         // MXFP4: [G][2F][d/2] packed E2M1
  const float* s13;      // [G][2F] FP8 channel scales (nullptr for MXFP4)
  const uint8_t* w2;     // [G][d][F]; MXFP4: [G][d][F/2]
  const float* s2;       // [G][d] (nullptr for MXFP4)
  const uint8_t* e13;    // MXFP4 E8M0 block scales [G][2F][d/32], else nullptr
  const uint8_t* e2;     // MXFP4 [G][d][F/32], else nullptr
  int w4;                // 1: MXFP4 weights
  const int32_t* offsets;  // device [G+1], or nullptr: one group of rows_fixed rows
  const int32_t* row_src;  // gather, nullptr = identity
  int src_div;
  int G;
  int F;
  int rows_fixed;
  int max_rows;          // upper bound of this set's rows
  uint8_t* h;            // [max_rows][F] FP8 codes (float32 on the f32 path)
  float* h_scale;        // [max_rows][F/128]
  void* out;             // [max_rows][d] bf16 (float32 on the f32 path)
};

struct FfnCall {
  int d;
  int a_rows;
  const void* a;         // [a_rows][d] FP8 codes or float32
  const float* a_scale;  // [a_rows]
  int nsets;             // 1 or 2
  FfnSet set[2];
};

// Optional per-step HIP events (start/stop per MOE_STEP_*), recorded around
// the kernels of each step.
struct StepEvents {
  void* const* start = nullptr;
  void* const* stop = nullptr;
  void mark(bool begin, int step, hipStream_t s) const {
    void* const* a = begin ? start : stop;
    if (a != nullptr && a[step] != nullptr) (void)hipEventRecord(static_cast<hipEvent_t>(a[step]), s);
  }
};

// Workspace for the tile lists of one call (both GEMMs), given the sets'
// row bounds; plus per-set h buffers sized by ffn_h_bytes.
size_t ffn_tiles_ws_bytes(const FfnCall& c);
size_t ffn_h_bytes(int max_rows, int F, bool fp8);
size_t ffn_hs_bytes(int max_rows, int F);
int choose_bm(int rows_hint);
hipError_t launch_ffn_tiles(const FfnCall& c, int bm, void* tiles_ws, hipStream_t s);
hipError_t launch_ffn_gemms(const FfnCall& c, int bm, void* tiles_ws, hipStream_t s,
                            const StepEvents& ev = StepEvents());
hipError_t launch_grouped_ffn_fp8(const FfnCall& c, void* tiles_ws, int rows_hint, hipStream_t s,
                                  const StepEvents& ev = StepEvents());
hipError_t launch_grouped_ffn_f32(const FfnCall& c, hipStream_t s,
                                  const StepEvents& ev = StepEvents());

// ----- combine --------------------------------------------------------------
hipError_t launch_combine_bf16(const uint16_t* expert_out, const int32_t* pair_to_row,
                               const float* w, const uint16_t* shared_out, uint16_t* y, int T,
                               int d, int k, hipStream_t s);
hipError_t launch_combine_f32(const float* expert_out, const int32_t* pair_to_row,
                              const float* w, const float* shared_out, float* y, int T, int d,
                              int k, hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
