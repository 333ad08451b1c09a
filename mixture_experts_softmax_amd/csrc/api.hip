// C ABI of libmoe: argument checks, workspace layout and kernel launches.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "common.h"
#include "internal.h"
#include "moe.h"

using namespace moe;

// Workspace of moe_layer_forward_noalloc: one copy per GPU, held from the
// library's load until the process ends. Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

bool is_dim(int v, int max) { return v >= MOE_DIM_ALIGN && v <= max && v % MOE_DIM_ALIGN == 0; }

moe_status_t check_shape(const moe_shape_t* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->T > MOE_MAX_T) return MOE_ERR_INVALID_ARG;
  if (!is_dim(s->d, MOE_MAX_D) || !is_dim(s->F, MOE_MAX_F)) return MOE_ERR_INVALID_ARG;
  if (s->F_shared != 0 && !is_dim(s->F_shared, MOE_MAX_F)) return MOE_ERR_INVALID_ARG;
  if (s->E < 1 || s->E > MOE_MAX_E) return MOE_ERR_INVALID_ARG;
  if (s->k < 1 || s->k > s->E || s->k > MOE_MAX_K) return MOE_ERR_INVALID_ARG;
  const bool fp8 = s->act_dtype == MOE_DTYPE_BF16 &&
                   (s->w_dtype == MOE_DTYPE_FP8_E4M3 || s->w_dtype == MOE_DTYPE_MXFP4);
  const bool f32 = s->act_dtype == MOE_DTYPE_F32 && s->w_dtype == MOE_DTYPE_F32;
  if (!fp8 && !f32) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The quantised path: bf16 activations, FP8 activation codes in the GEMMs,
// FP8 or MXFP4 weights.
bool is_fp8(const moe_shape_t* s) { return s->w_dtype != MOE_DTYPE_F32; }
bool is_w4(int w_dtype) { return w_dtype == MOE_DTYPE_MXFP4; }

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool al256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Bump allocator over a caller-provided workspace (256-byte aligned regions).
struct Carve {
  uint8_t* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base == nullptr ? nullptr : base + off);
    off += align_up(bytes, 256);
    return p;
  }
};

moe_status_t check_ffn(const moe_ffn_t* f) {
  if (f == nullptr) return MOE_ERR_INVALID_ARG;
  if (!is_dim(f->d, MOE_MAX_D) || !is_dim(f->F, MOE_MAX_F)) return MOE_ERR_INVALID_ARG;
  if (f->num_groups < 1 || f->num_groups > 1023) return MOE_ERR_INVALID_ARG;
  if (f->max_rows < 0 || f->max_rows > MOE_MAX_T * MOE_MAX_K) return MOE_ERR_INVALID_ARG;
  if (f->src_div < 1 || f->a_rows < 0) return MOE_ERR_INVALID_ARG;
  if (f->w_dtype != MOE_DTYPE_FP8_E4M3 && f->w_dtype != MOE_DTYPE_MXFP4 &&
      f->w_dtype != MOE_DTYPE_F32)
    return MOE_ERR_UNSUPPORTED;
  if (f->max_rows == 0) return MOE_OK;
  if (f->a_rows < 1) return MOE_ERR_INVALID_ARG;
  if (!f->group_offsets || !f->a || !f->w13 || !f->w2 || !f->out) return MOE_ERR_INVALID_ARG;
  if (!al16(f->a) || !al16(f->w13) || !al16(f->w2) || !al16(f->out) || !al16(f->h_out))
    return MOE_ERR_INVALID_ARG;
  if (f->w_dtype != MOE_DTYPE_F32 && (!f->a_scale || !f->w13_scale || !f->w2_scale))
    return MOE_ERR_INVALID_ARG;
  if (is_w4(f->w_dtype) && (!al16(f->w13_scale) || !al16(f->w2_scale)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Weight pointers of one set; scales are float32 channel scales (FP8) or E8M0
// block-scale bytes (MXFP4, w4).
FfnSet make_set(const void* w13, const void* s13, const void* w2, const void* s2, bool w4,
                const int32_t* offsets, const int32_t* row_src, int src_div, int G, int F,
                int rows_fixed, int max_rows, void* out) {
  FfnSet S{};
  S.w13 = static_cast<const uint8_t*>(w13);
  S.w2 = static_cast<const uint8_t*>(w2);
  S.w4 = w4 ? 1 : 0;
  if (w4) {
    S.e13 = static_cast<const uint8_t*>(s13);
    S.e2 = static_cast<const uint8_t*>(s2);
  } else {
    S.s13 = static_cast<const float*>(s13);
    S.s2 = static_cast<const float*>(s2);
  }
  S.offsets = offsets;
  S.row_src = row_src;
  S.src_div = src_div;
  S.G = G;
  S.F = F;
  S.rows_fixed = rows_fixed;
  S.max_rows = max_rows;
  S.out = out;
  return S;
}

// Lays out (and, with a real base, assigns) the per-set h buffers and the tile
// lists of one grouped-FFN call; returns the bytes used.
size_t carve_ffn(FfnCall& c, bool fp8, Carve& cv, void** tiles) {
  for (int i = 0; i < c.nsets; ++i) {
    FfnSet& S = c.set[i];
    S.h = cv.take<uint8_t>(ffn_h_bytes(S.max_rows, S.F, fp8));
    S.h_scale = fp8 ? cv.take<float>(ffn_hs_bytes(S.max_rows, S.F)) : nullptr;
  }
  *tiles = fp8 ? cv.take<uint8_t>(ffn_tiles_ws_bytes(c)) : nullptr;
  return cv.off;
}

// The routed experts alone (set 0) and the shared expert alone (set 1 as the
// only set) of a layer's grouped-FFN call.
FfnCall routed_call(const FfnCall& c) {
  FfnCall r = c;
  r.nsets = 1;
  return r;
}
FfnCall shared_call(const FfnCall& c) {
  FfnCall r = c;
  r.nsets = 1;
  r.set[0] = c.set[1];
  return r;
}

// The layer's workspace; with base == nullptr only the size is computed.
struct LayerWs {
  int32_t* ids;
  float* w;
  uint8_t* xq;
  float* xs;
  float* logits;
  uint64_t* masks;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_to_row;
  void* expert_out;
  void* shared_out;
  void* tiles;
  void* tiles_shared;  // the shared expert's own tile lists (second-stream schedule)
  size_t bytes;
};

LayerWs layer_ws(const moe_shape_t* s, void* base, FfnCall* call) {
  const bool fp8 = is_fp8(s);
  const size_t T = s->T, k = s->k, d = s->d, E = s->E;
  const size_t ob = fp8 ? 2 : 4;
  Carve cv(base);
  LayerWs L{};
  L.ids = cv.take<int32_t>(T * k * 4);
  L.w = cv.take<float>(T * k * 4);
  L.xq = fp8 ? cv.take<uint8_t>(T * d) : nullptr;
  L.xs = fp8 ? cv.take<float>(T * 4) : nullptr;
  L.logits = cv.take<float>(route_ws_bytes(s->T, s->d, s->E));
  L.masks = cv.take<uint64_t>(perm_masks_bytes(s->T, s->E));
  L.counts = cv.take<int32_t>(perm_counts_bytes(s->T, s->E));
  L.offsets = cv.take<int32_t>((E + 1) * 4);
  L.sorted_pair = cv.take<int32_t>(T * k * 4);
  L.pair_to_row = cv.take<int32_t>(T * k * 4);
  L.expert_out = cv.take<uint8_t>(T * k * d * ob);
  L.shared_out = s->F_shared > 0 ? cv.take<uint8_t>(T * d * ob) : nullptr;
  FfnCall c{};
  c.d = s->d;
  c.nsets = s->F_shared > 0 ? 2 : 1;
  const bool w4 = is_w4(s->w_dtype);
  c.set[0] = make_set(nullptr, nullptr, nullptr, nullptr, w4, L.offsets, L.sorted_pair, s->k,
                      s->E, s->F, 0, s->T * s->k, L.expert_out);
  if (c.nsets > 1)
    c.set[1] = make_set(nullptr, nullptr, nullptr, nullptr, w4, nullptr, nullptr, 1, 1,
                        s->F_shared, s->T, s->T, L.shared_out);
  carve_ffn(c, fp8, cv, &L.tiles);
  L.tiles_shared = nullptr;
  if (fp8 && c.nsets > 1) {
    FfnCall cs = shared_call(c);
    L.tiles_shared = cv.take<uint8_t>(ffn_tiles_ws_bytes(cs));
  }
  L.bytes = cv.off;
  if (call) *call = c;
  return L;
}

// Pointers and alignment of a layer call (shape already checked, T > 0).
moe_status_t check_layer_args(const moe_shape_t* s, const moe_weights_t* wt, const void* x,
                              const void* y) {
  if (!wt || !x || !y || !wt->w_router || !wt->w13 || !wt->w2) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(y) || !al16(wt->w_router) || !al16(wt->w13) || !al16(wt->w2))
    return MOE_ERR_INVALID_ARG;
  if (s->F_shared > 0 && (!al16(wt->ws13) || !al16(wt->ws2))) return MOE_ERR_INVALID_ARG;
  const bool fp8 = is_fp8(s);
  if (fp8 && (!wt->w13_scale || !wt->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (s->F_shared > 0 && (!wt->ws13 || !wt->ws2 || (fp8 && (!wt->ws13_scale || !wt->ws2_scale))))
    return MOE_ERR_INVALID_ARG;
  if (is_w4(s->w_dtype) && (!al16(wt->w13_scale) || !al16(wt->w2_scale) ||
                            (s->F_shared > 0 && (!al16(wt->ws13_scale) || !al16(wt->ws2_scale)))))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_qk(const moe_qk_shape_t* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_DTYPE_BF16 && s->dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (s->T < 0 || s->T > MOE_MAX_T) return MOE_ERR_INVALID_ARG;
  if (s->n_q < 0 || s->n_kv < 0 || s->n_q + s->n_kv < 1 || s->n_q + s->n_kv > 256)
    return MOE_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return MOE_ERR_INVALID_ARG;
  if (s->style != MOE_ROPE_INTERLEAVED && s->style != MOE_ROPE_HALVES) return MOE_ERR_INVALID_ARG;
  if (!(s->eps >= 0.f) || !std::isfinite(s->eps)) return MOE_ERR_INVALID_ARG;
  if (!(s->theta > 0.f) || !std::isfinite(s->theta)) return MOE_ERR_INVALID_ARG;
  const int64_t vec = s->dtype == MOE_DTYPE_BF16 ? 8 : 4;  // elements per 16 bytes
  if (s->row_stride < 1 || s->q_offset < 0 || s->k_offset < 0) return MOE_ERR_INVALID_ARG;
  if (s->row_stride % vec || s->q_offset % vec || s->k_offset % vec) return MOE_ERR_INVALID_ARG;
  const int64_t qe = s->q_offset + (int64_t)s->n_q * s->head_dim;
  const int64_t ke = s->k_offset + (int64_t)s->n_kv * s->head_dim;
  if (qe > s->row_stride || ke > s->row_stride) return MOE_ERR_INVALID_ARG;
  if (s->n_q > 0 && s->n_kv > 0 && s->q_offset < ke && s->k_offset < qe) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_qk_norm_rope(const moe_qk_shape_t* s, void* qkv, const int32_t* positions,
                              const void* q_weight, const void* k_weight, void* stream) {
  const moe_status_t st = check_qk(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!qkv || !positions || (s->n_q > 0 && !q_weight) || (s->n_kv > 0 && !k_weight))
    return MOE_ERR_INVALID_ARG;
  if (!al16(qkv) || !al16(q_weight) || !al16(k_weight)) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_qk_norm_rope(*s, qkv, positions, q_weight, k_weight,
                                      static_cast<hipStream_t>(stream)));
}

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH:
      return "shape needs more workspace than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

moe_status_t moe_check_shape(const moe_shape_t* shape) { return check_shape(shape); }

moe_status_t moe_layer_workspace_size(const moe_shape_t* shape, size_t* bytes) {
  const moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = layer_ws(shape, nullptr, nullptr).bytes;
  return MOE_OK;
}

moe_status_t moe_layer_workspace_regions(const moe_shape_t* shape, moe_layer_regions_t* r) {
  const moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (r == nullptr) return MOE_ERR_INVALID_ARG;
  // laid out against a base far from zero, so that a region at offset 0
  // cannot be mistaken for a missing one
  uint8_t* const base = reinterpret_cast<uint8_t*>(uintptr_t(1) << 40);
  FfnCall c;
  const LayerWs L = layer_ws(shape, base, &c);
  auto off = [&](const void* p) {
    return p == nullptr ? MOE_NO_REGION : (size_t)(static_cast<const uint8_t*>(p) - base);
  };
  const bool fp8 = is_fp8(shape);
  r->xq = off(L.xq);
  r->x_scale = off(L.xs);
  r->offsets = off(L.offsets);
  r->sorted_pair = off(L.sorted_pair);
  r->pair_to_row = off(L.pair_to_row);
  r->h = off(c.set[0].h);
  r->h_scale = fp8 ? off(c.set[0].h_scale) : MOE_NO_REGION;
  r->h_shared = c.nsets > 1 ? off(c.set[1].h) : MOE_NO_REGION;
  r->h_shared_scale = (c.nsets > 1 && fp8) ? off(c.set[1].h_scale) : MOE_NO_REGION;
  r->expert_out = off(L.expert_out);
  r->shared_out = off(L.shared_out);
  return MOE_OK;
}

// The router's workspace: the K-split partial logits, then the tile masks
// (written when tile counts are requested).
static size_t route_call_ws_bytes(const moe_shape_t* s) {
  return route_ws_bytes(s->T, s->d, s->E) + perm_masks_bytes(s->T, s->E);
}

moe_status_t moe_route_workspace_size(const moe_shape_t* shape, size_t* bytes) {
  const moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = route_call_ws_bytes(shape);
  return MOE_OK;
}

moe_status_t moe_permute_workspace_size(const moe_shape_t* shape, size_t* bytes) {
  const moe_status_t st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = permute_ws_bytes(shape->T, shape->E);
  return MOE_OK;
}

static FfnCall ffn_call(const moe_ffn_t* f) {
  FfnCall c{};
  c.d = f->d;
  c.a_rows = f->a_rows;
  c.a = f->a;
  c.a_scale = f->a_scale;
  c.nsets = 1;
  c.set[0] = make_set(f->w13, f->w13_scale, f->w2, f->w2_scale, is_w4(f->w_dtype),
                      f->group_offsets, f->row_src, f->src_div, f->num_groups, f->F, 0,
                      f->max_rows, f->out);
  return c;
}

moe_status_t moe_grouped_ffn_workspace_size(const moe_ffn_t* ffn, size_t* bytes) {
  const moe_status_t st = check_ffn(ffn);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  FfnCall c = ffn_call(ffn);
  Carve cv(nullptr);
  void* tiles;
  *bytes = carve_ffn(c, ffn->w_dtype != MOE_DTYPE_F32, cv, &tiles);
  return MOE_OK;
}

moe_status_t moe_route_topk(const moe_shape_t* s, const void* x, const void* w_router,
                            const float* router_bias, int32_t* topk_ids, float* topk_w,
                            uint8_t* xq, float* x_scale, int32_t* tile_counts, void* workspace,
                            size_t workspace_bytes, void* stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(w_router)) return MOE_ERR_INVALID_ARG;
  const bool fp8 = is_fp8(s);
  if (fp8 && (!xq || !x_scale || !al16(xq))) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < route_call_ws_bytes(s) || !al256(workspace))
    return MOE_ERR_WORKSPACE;
  uint64_t* masks = tile_counts == nullptr
                        ? nullptr
                        : reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) +
                                                      route_ws_bytes(s->T, s->d, s->E));
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = launch_route(fp8, x, w_router, router_bias, s->T, s->d, s->E, s->k, topk_ids,
                              topk_w, fp8 ? xq : nullptr, fp8 ? x_scale : nullptr, workspace,
                              masks, nullptr, nullptr, hs);
  if (e == hipSuccess && tile_counts != nullptr)
    e = launch_tile_counts(masks, s->T, s->E, tile_counts, hs);
  return from_hip(e);
}

moe_status_t moe_permute(const moe_shape_t* s, const int32_t* topk_ids, const uint8_t* xq,
                         const float* x_scale, int32_t* offsets, int32_t* sorted_pair,
                         int32_t* pair_to_row, uint8_t* x_perm, float* x_perm_scale,
                         int32_t* tile_counts, void* workspace, size_t workspace_bytes,
                         void* stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!topk_ids || !offsets || !sorted_pair || !pair_to_row) return MOE_ERR_INVALID_ARG;
  // the gather: all four pointers (quantised paths only) or none
  const int ng = (xq != nullptr) + (x_scale != nullptr) + (x_perm != nullptr) +
                 (x_perm_scale != nullptr);
  if (ng != 0 && (ng != 4 || !is_fp8(s) || !al16(xq) || !al16(x_perm)))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < permute_ws_bytes(s->T, s->E) || !al256(workspace))
    return MOE_ERR_WORKSPACE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = launch_permute(topk_ids, s->T, s->E, s->k, offsets, sorted_pair, pair_to_row,
                                tile_counts, workspace, hs);
  if (e == hipSuccess && ng == 4)
    e = launch_perm_gather(xq, x_scale, sorted_pair, offsets, s->T, s->E, s->k, s->d, x_perm,
                           x_perm_scale, hs);
  return from_hip(e);
}

moe_status_t moe_grouped_ffn(const moe_ffn_t* f, void* workspace, size_t workspace_bytes,
                             void* stream) {
  moe_status_t st = check_ffn(f);
  if (st != MOE_OK) return st;
  if (f->max_rows == 0) return MOE_OK;
  const bool fp8 = f->w_dtype != MOE_DTYPE_F32;
  FfnCall c = ffn_call(f);
  {
    Carve probe(nullptr);
    void* t;
    const size_t need = carve_ffn(c, fp8, probe, &t);
    if (!workspace || workspace_bytes < need || !al256(workspace)) return MOE_ERR_WORKSPACE;
  }
  Carve cv(workspace);
  void* tiles = nullptr;
  carve_ffn(c, fp8, cv, &tiles);
  if (f->h_out != nullptr) c.set[0].h = static_cast<uint8_t*>(f->h_out);
  if (fp8 && f->h_scale_out != nullptr) c.set[0].h_scale = f->h_scale_out;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (fp8) {
    const int hint = ceil_div(f->max_rows, f->num_groups);
    return from_hip(launch_grouped_ffn_fp8(c, tiles, hint, hs));
  }
  return from_hip(launch_grouped_ffn_f32(c, hs));
}

moe_status_t moe_combine(const moe_shape_t* s, const void* expert_out,
                         const int32_t* pair_to_row, const float* topk_w,
                         const void* shared_out, void* y, void* stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!expert_out || !pair_to_row || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!al16(expert_out) || !al16(y) || (shared_out && !al16(shared_out))) return MOE_ERR_INVALID_ARG;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (is_fp8(s))
    return from_hip(launch_combine_bf16(static_cast<const uint16_t*>(expert_out), pair_to_row,
                                        topk_w, static_cast<const uint16_t*>(shared_out),
                                        static_cast<uint16_t*>(y), s->T, s->d, s->k, hs));
  return from_hip(launch_combine_f32(static_cast<const float*>(expert_out), pair_to_row, topk_w,
                                     static_cast<const float*>(shared_out),
                                     static_cast<float*>(y), s->T, s->d, s->k, hs));
}

moe_status_t moe_layer_forward(const moe_shape_t* s, const moe_weights_t* wt, const void* x,
                               void* y, int32_t* topk_ids, float* topk_w, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return moe_layer_forward_events(s, wt, x, y, topk_ids, topk_w, workspace, workspace_bytes,
                                  stream, nullptr, nullptr);
}

// The layer on `stream`; with side != nullptr (quantised paths with a shared
// expert) the shared expert's GEMMs run on `side`, forked by `fork` right after
// the router's logits launch and joined by `join` before the combine.
static moe_status_t layer_forward(const moe_shape_t* s, const moe_weights_t* wt, const void* x,
                                  void* y, int32_t* topk_ids, float* topk_w, void* workspace,
                                  size_t workspace_bytes, hipStream_t hs, const StepEvents& ev,
                                  hipStream_t side, hipEvent_t fork, hipEvent_t join) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  st = check_layer_args(s, wt, x, y);
  if (st != MOE_OK) return st;
  const bool fp8 = is_fp8(s);
  const bool w4 = is_w4(s->w_dtype);
  const size_t need = layer_ws(s, nullptr, nullptr).bytes;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return MOE_ERR_WORKSPACE;

  FfnCall c;
  LayerWs L = layer_ws(s, workspace, &c);
  int32_t* ids = topk_ids ? topk_ids : L.ids;
  float* w = topk_w ? topk_w : L.w;

  c.a_rows = s->T;
  c.a = fp8 ? static_cast<const void*>(L.xq) : x;
  c.a_scale = L.xs;
  auto set_weights = [&](FfnSet& S, const void* w13, const void* s13, const void* w2,
                         const void* s2) {
    S = make_set(w13, s13, w2, s2, w4, S.offsets, S.row_src, S.src_div, S.G, S.F, S.rows_fixed,
                 S.max_rows, S.out);
  };
  {
    FfnSet& R = c.set[0];
    uint8_t* h = R.h;
    float* hsc = R.h_scale;
    set_weights(R, wt->w13, wt->w13_scale, wt->w2, wt->w2_scale);
    R.h = h;
    R.h_scale = hsc;
  }
  if (c.nsets > 1) {
    FfnSet& Sh = c.set[1];
    uint8_t* h = Sh.h;
    float* hsc = Sh.h_scale;
    set_weights(Sh, wt->ws13, wt->ws13_scale, wt->ws2, wt->ws2_scale);
    Sh.h = h;
    Sh.h_scale = hsc;
  }
  const int bm = choose_bm(ceil_div(s->T * s->k, s->E));
  // second-stream schedule: the routed launches carry set 0 only, the shared
  // expert (same tile height, so the same kernels and tiles) runs on `side`
  const bool split = side != nullptr && fp8 && c.nsets > 1;
  const FfnCall cr = split ? routed_call(c) : c;

  // Up to one permutation tile of tokens, the top-k workgroup also does the
  // permutation (and, FP8 path, writes the FFN tile lists); the permute step
  // then has no kernels of its own.
  const bool fused = s->T <= kPermTile;
  RoutePermute rp{L.offsets, L.sorted_pair, L.pair_to_row, fp8 ? &cr : nullptr, bm,
                  fp8 ? L.tiles : nullptr};
  // Above one permutation tile (single stream) x is quantised by the scan
  // launch, whose one scanning workgroup leaves the other CUs idle; with
  // the second stream the shared expert needs the codes right after the
  // logits, so the logits launch writes them.
  const bool quant_in_scan = fp8 && !fused && !split;
  hipError_t e;
  ev.mark(true, MOE_STEP_ROUTE, hs);
  e = launch_route(fp8, x, wt->w_router, wt->router_bias, s->T, s->d, s->E, s->k, ids, w,
                   quant_in_scan ? nullptr : L.xq, L.xs, L.logits, L.masks, L.counts,
                   fused ? &rp : nullptr, hs, split ? fork : nullptr);
  ev.mark(false, MOE_STEP_ROUTE, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (split) {  // the shared expert needs only the x codes
    const FfnCall csh = shared_call(c);
    e = hipStreamWaitEvent(side, fork, 0);
    if (e == hipSuccess) e = launch_ffn_tiles(csh, bm, L.tiles_shared, side);
    if (e == hipSuccess) e = launch_ffn_gemms(csh, bm, L.tiles_shared, side);
    if (e == hipSuccess) e = hipEventRecord(join, side);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  // scan + scatter; on the FP8 path the scan also writes the FFN tile lists
  ev.mark(true, MOE_STEP_PERMUTE, hs);
  const QuantRows qr{static_cast<const uint16_t*>(x), s->T, s->d, L.xq, L.xs};
  if (!fused)
    e = launch_perm_scan_scatter(ids, s->T, s->E, s->k, L.masks, L.counts, L.offsets,
                                 L.sorted_pair, L.pair_to_row, fp8 ? &cr : nullptr, bm,
                                 fp8 ? L.tiles : nullptr, hs, quant_in_scan ? &qr : nullptr);
  ev.mark(false, MOE_STEP_PERMUTE, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;

  if (fp8)
    e = launch_ffn_gemms(cr, bm, L.tiles, hs, ev);
  else
    e = launch_grouped_ffn_f32(c, hs, ev);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (split && hipStreamWaitEvent(hs, join, 0) != hipSuccess) return MOE_ERR_HIP;

  ev.mark(true, MOE_STEP_COMBINE, hs);
  if (fp8)
    e = launch_combine_bf16(static_cast<const uint16_t*>(L.expert_out), L.pair_to_row, w,
                            static_cast<const uint16_t*>(L.shared_out), static_cast<uint16_t*>(y),
                            s->T, s->d, s->k, hs);
  else
    e = launch_combine_f32(static_cast<const float*>(L.expert_out), L.pair_to_row, w,
                           static_cast<const float*>(L.shared_out), static_cast<float*>(y), s->T,
                           s->d, s->k, hs);
  ev.mark(false, MOE_STEP_COMBINE, hs);
  return from_hip(e);
}

moe_status_t moe_layer_forward_events(const moe_shape_t* s, const moe_weights_t* wt,
                                      const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* start_events, void* const* stop_events) {
  StepEvents ev;
  ev.start = start_events;
  ev.stop = stop_events;
  return layer_forward(s, wt, x, y, topk_ids, topk_w, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), ev, nullptr, nullptr, nullptr);
}

moe_status_t moe_layer_forward_overlap(const moe_shape_t* s, const moe_weights_t* wt,
                                       const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       void* side_stream, void* fork_event, void* join_event) {
  if (side_stream == nullptr || side_stream == stream || fork_event == nullptr ||
      join_event == nullptr || fork_event == join_event)
    return MOE_ERR_INVALID_ARG;
  return layer_forward(s, wt, x, y, topk_ids, topk_w, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), StepEvents(),
                       static_cast<hipStream_t>(side_stream), static_cast<hipEvent_t>(fork_event),
                       static_cast<hipEvent_t>(join_event));
}

moe_status_t moe_layer_forward_noalloc(const moe_shape_t* s, const moe_weights_t* wt,
                                       const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                       void* stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  st = check_layer_args(s, wt, x, y);
  if (st != MOE_OK) return st;
  if (layer_ws(s, nullptr, nullptr).bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_layer_forward_events(s, wt, x, y, topk_ids, topk_w, ws, MOE_NOALLOC_SCRATCH_BYTES,
                                  stream, nullptr, nullptr);
}

void moe_host_e4m3_encode(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = moe::e4m3_encode(in[i]);
}

}  // extern "C"
