/*
 * moe.h -- C ABI of libmoe, the forward pass of one mixture-of-experts layer
 * with softmax top-k gating, SwiGLU experts stored in FP8 and one always-on
 * shared expert, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The layer follows the model described on the NVIDIA blog "How NVIDIA extreme
 * hardware-software co-design delivered a large inference boost for Sarvam
 * AI's sovereign models" (section "Scaling multilingual sovereign AI with
 * MoE": 128 routed experts, top-6 or top-8 routing, a shared expert beside the
 * routed ones; Table 1: router logits and top-k as one fused step, routed
 * experts as grouped GEMMs, the shared expert as a separate computation).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory (or memory
 *    the device can access) owned by the caller; the library never allocates,
 *    frees or synchronises inside these calls and keeps no global state, so
 *    calls on different streams do not interfere unless their buffers alias.
 *    The one exception is moe_layer_forward_noalloc, whose workspace is a
 *    static buffer of the library (one per GPU), declared last below.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *    work and return; results are ready when the stream reaches them.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    rejected call returns a negative status and enqueues nothing. A failed
 *    launch returns MOE_ERR_HIP.
 *  - All arrays are dense and row-major; weight matrices are [out][in].
 *    Activation, weight and output arrays must start on a 16-byte boundary
 *    and workspaces on a 256-byte boundary (MOE_ERR_INVALID_ARG /
 *    MOE_ERR_WORKSPACE otherwise).
 *  - Inputs are assumed finite; results for NaN or Inf inputs are unspecified.
 *  - T == 0 is valid and enqueues nothing.
 *
 * Supported precisions (moe_shape_t.act_dtype, .w_dtype):
 *  - (MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3): bf16 activations and router weight,
 *    OCP FP8 E4M3 expert weights with one float32 scale per output channel,
 *    bf16 output. Activations entering the expert GEMMs are quantised to FP8
 *    E4M3: x per token, the SwiGLU output h per (row, 128-column block), each
 *    with a float32 scale amax/448 (1.0 for an all-zero block), codes rounded
 *    to nearest even with saturation at +-448.
 *  - (MOE_DTYPE_BF16, MOE_DTYPE_MXFP4): as the FP8 path, with OCP
 *    Microscaling MXFP4 expert weights (the analogue of the NVFP4 weights the
 *    NVIDIA blog runs on Blackwell, section "Running on Blackwell"): E2M1
 *    elements packed two per byte along the reduction dimension (element 2i in
 *    the low nibble of byte i) with one E8M0 scale byte (value 2^(e - 127)) per
 *    32 elements, and no channel scale:
 *      w13 [E][2F][d/2] bytes, w13_scale [E][2F][d/32] bytes,
 *      w2  [E][d][F/2],        w2_scale  [E][d][F/32],
 *    the shared expert likewise without the E dimension. A weight's value is
 *    its E2M1 value times its block's scale.
 *  - (MOE_DTYPE_F32, MOE_DTYPE_F32): float32 throughout, no quantisation.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

/* Limits checked by every entry point. */
#define MOE_MAX_E 256      /* routed experts */
#define MOE_MAX_K 16       /* experts per token */
#define MOE_MAX_D 16384    /* hidden size */
#define MOE_MAX_F 16384    /* expert FFN width */
#define MOE_MAX_T (1 << 22)
#define MOE_DIM_ALIGN 128  /* d, F and F_shared must be multiples of this */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size or shape */
  MOE_ERR_UNSUPPORTED = -2, /* unsupported (act_dtype, w_dtype) pair */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4,         /* the HIP runtime reported an error */
  MOE_ERR_SCRATCH = -5      /* the shape needs more than moe_layer_forward_noalloc's
                               static scratch (MOE_NOALLOC_SCRATCH_BYTES) */
} moe_status_t;

typedef enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_FP8_E4M3 = 2,
  MOE_DTYPE_MXFP4 = 3       /* expert weights only */
} moe_dtype_t;

/* Shape of one layer call. */
typedef struct moe_shape {
  int32_t T;         /* tokens in this call, 0 <= T <= MOE_MAX_T */
  int32_t d;         /* hidden size */
  int32_t E;         /* routed experts, 1..MOE_MAX_E */
  int32_t k;         /* experts chosen per token, 1..min(E, MOE_MAX_K) */
  int32_t F;         /* routed expert FFN width */
  int32_t F_shared;  /* shared expert FFN width; 0 = no shared expert */
  int32_t act_dtype; /* moe_dtype_t of x, the router weight and y */
  int32_t w_dtype;   /* moe_dtype_t of the expert weights */
} moe_shape_t;

/* The layer's weights (device pointers). */
typedef struct moe_weights {
  const void* w_router;     /* [E][d], act_dtype */
  const float* router_bias; /* [E] added to the logits before softmax, or NULL */
  const void* w13;          /* [E][2F][d], w_dtype; rows 0..F-1 gate, F..2F-1 up */
  const void* w13_scale;    /* FP8: float32 [E][2F] per-output-row scales; MXFP4: E8M0
                               bytes [E][2F][d/32]; F32: NULL */
  const void* w2;           /* [E][d][F], w_dtype */
  const void* w2_scale;     /* FP8: float32 [E][d]; MXFP4: E8M0 bytes [E][d][F/32] */
  const void* ws13;         /* shared expert [2F_shared][d] (NULL if F_shared == 0) */
  const void* ws13_scale;   /* FP8: float32 [2F_shared]; MXFP4: bytes [2F_shared][d/32] */
  const void* ws2;          /* shared expert [d][F_shared] */
  const void* ws2_scale;    /* FP8: float32 [d]; MXFP4: bytes [d][F_shared/32] */
} moe_weights_t;

/* One grouped SwiGLU FFN call: G groups of rows, each group g multiplying its
 * rows by its own expert's weights. */
typedef struct moe_ffn {
  int32_t d;                    /* hidden size (multiple of 128) */
  int32_t F;                    /* FFN width of every group (multiple of 128) */
  int32_t num_groups;           /* G >= 1 */
  int32_t max_rows;             /* rows of `out`; group_offsets[G] must not exceed it */
  int32_t w_dtype;              /* MOE_DTYPE_FP8_E4M3, MOE_DTYPE_MXFP4 or MOE_DTYPE_F32 */
  const int32_t* group_offsets; /* device [G+1], non-decreasing, [0] == 0: group g owns
                                   grouped rows group_offsets[g] .. group_offsets[g+1]-1 */
  const int32_t* row_src;       /* device [max_rows] or NULL: grouped row r reads activation
                                   row row_src[r] / src_div (NULL: activation row r) */
  int32_t src_div;              /* >= 1 */
  int32_t a_rows;               /* rows of `a`; every source row must be below it */
  const void* a;                /* [a_rows][d]: FP8 codes (FP8, MXFP4 paths) or float32 */
  const float* a_scale;         /* [a_rows] per-row scales (FP8/MXFP4 paths), else NULL */
  const void* w13;              /* [G][2F][d] (MXFP4: [G][2F][d/2] packed) */
  const void* w13_scale;        /* FP8: float32 [G][2F]; MXFP4: E8M0 bytes [G][2F][d/32] */
  const void* w2;               /* [G][d][F] (MXFP4: [G][d][F/2] packed) */
  const void* w2_scale;         /* FP8: float32 [G][d]; MXFP4: E8M0 bytes [G][d][F/32] */
  void* out;                    /* [max_rows][d]: bf16 (FP8, MXFP4 paths) or float32 */
  void* h_out;                  /* optional: receives h, [max_rows][F] FP8 codes (FP8, MXFP4)
                                   or float32; NULL keeps h in the workspace */
  float* h_scale_out;           /* optional: [max_rows][F/128] block scales of h (FP8, MXFP4) */
} moe_ffn_t;

/* ABI version (MOE_ABI_VERSION) and a static text for a status code. */
int32_t moe_abi_version(void);
const char* moe_status_string(int32_t status);

/* Checks a layer shape against the limits above. */
moe_status_t moe_check_shape(const moe_shape_t* shape);

/* Workspace sizes in bytes (host-only queries, nothing is enqueued). */
moe_status_t moe_layer_workspace_size(const moe_shape_t* shape, size_t* bytes);
moe_status_t moe_route_workspace_size(const moe_shape_t* shape, size_t* bytes);
moe_status_t moe_permute_workspace_size(const moe_shape_t* shape, size_t* bytes);
moe_status_t moe_grouped_ffn_workspace_size(const moe_ffn_t* ffn, size_t* bytes);

/*
 * Router: logits, softmax, top-k selection and renormalised gate weights
 * (NVIDIA blog, Table 1 row "Router logits and TopK" and the
 * paragraph on MoE routing; peacm.com repost section 3.1: the fused router
 * writes integer expert indices and float scores; ijyty.com "InferX" page
 * section 2.4: softmax over the expert logits, then top-k).
 *
 *   l[t, e]  = sum_i x[t, i] * w_router[e, i] + router_bias[e]   (float32 accumulation;
 *              on the bf16 path split over K, the slices summed in slice order)
 *   ids[t]   = the k experts with the largest l[t, .], largest first, equal
 *              logits ordered by lower expert index
 *   w[t, j]  = softmax(l[t, .])[ids[t, j]] / sum_j' softmax(l[t, .])[ids[t, j']]
 *
 * x [T][d] and w_router [E][d] in act_dtype; router_bias [E] float32 or NULL.
 * Outputs topk_ids [T][k] int32 and topk_w [T][k] float32. On the FP8 and MXFP4
 * paths (bf16 activations) the
 * logits launch also writes xq [T][d] (FP8 E4M3 codes of x / x_scale[t]) and
 * x_scale [T] (amax of row t over 448, 1.0 for a zero row); both are required
 * there and ignored on the float32 path.
 * tile_counts (optional, NULL to skip): int32 [ceil(T/64)][E], the number of
 * tokens of each 64-token tile routed to each expert (the permutation's
 * histogram, taken from the selection kernel's per-tile expert masks; one more
 * small launch when requested). Two launches otherwise (logits, selection).
 * Needs a workspace of moe_route_workspace_size() bytes (the float32 partial
 * logits of the K slices and the tile masks).
 */
moe_status_t moe_route_topk(const moe_shape_t* shape, const void* x, const void* w_router,
                            const float* router_bias, int32_t* topk_ids, float* topk_w,
                            uint8_t* xq, float* x_scale, int32_t* tile_counts, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Permutation of the T*k (token, slot) pairs into expert-contiguous order (the
 * scatter that the InferX page, section 3.3, fuses after its top-k router:
 * moe_scatter moves each token's row to the rows of its chosen experts).
 * Pair p = t*k + j. Rows of expert e are offsets[e] .. offsets[e+1]-1, pairs
 * of one expert in ascending token order:
 *   offsets     [E+1]  offsets[0] = 0, offsets[E] = number of valid pairs
 *   sorted_pair [T*k]  row -> pair
 *   pair_to_row [T*k]  pair -> row
 *   tile_counts [ceil(T/64)][E] int32 (optional, NULL to skip): tokens of each
 *               64-token tile routed to each expert (the histogram)
 * Gather (optional; on the quantised paths, all four pointers or none):
 *   x_perm       [T*k][d] bytes: x_perm[row] = xq[sorted_pair[row] / k]
 *   x_perm_scale [T*k] float32:  x_scale[sorted_pair[row] / k]
 * from xq [T][d] FP8 codes and x_scale [T] (as moe_route_topk writes them);
 * only rows below offsets[E] are written. The result is moe_grouped_ffn's
 * activation input with row_src = NULL. moe_layer_forward does not materialise
 * it: its GEMMs read the rows of xq through sorted_pair while staging them.
 * topk_ids must hold values in [0, E), distinct within a token; a pair with an
 * id outside [0, E) gets no row and pair_to_row = -1. Needs a workspace of
 * moe_permute_workspace_size() bytes.
 */
moe_status_t moe_permute(const moe_shape_t* shape, const int32_t* topk_ids, const uint8_t* xq,
                         const float* x_scale, int32_t* offsets, int32_t* sorted_pair,
                         int32_t* pair_to_row, uint8_t* x_perm, float* x_perm_scale,
                         int32_t* tile_counts, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Grouped SwiGLU expert FFN (NVIDIA blog, section "Performance challenges":
 * routed experts run as grouped GEMM kernels with the expert weights resident
 * in HBM; Table 1 rows "Routed expert compute" and "Shared expert compute").
 * For grouped row r of group g with activation row s:
 *   FP8 path:  gu[n] = a_scale[s] * w13_scale[g][n] * sum_i a[s][i] * w13[g][n][i]
 *              h[n]  = silu(gu[n]) * gu[F + n],  silu(z) = z / (1 + exp(-z))
 *              h is quantised per 128-column block (scale amax/448, E4M3 codes)
 *              out[r][m] = w2_scale[g][m] * sum_b s_h[b] * sum_{n in b} hq[n] * w2[g][m][n]
 *              out is rounded to bf16 (nearest even)
 *   MXFP4:     as the FP8 path with w13[g][n][i] and w2[g][m][n] the decoded
 *              MXFP4 values (E2M1 value times 2^(block scale - 127)) and no
 *              w13_scale / w2_scale factor.
 *   F32 path:  the same without any quantisation, float32 out.
 * Rows beyond group_offsets[G] are not written. Needs a workspace of
 * moe_grouped_ffn_workspace_size() bytes. The shared expert is one group over
 * all tokens (row_src = NULL).
 */
moe_status_t moe_grouped_ffn(const moe_ffn_t* ffn, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Gate-weighted combine (ijyty.com "InferX" page, section 3.3: the experts'
 * rows of a token are brought back and added with the router's weights; the
 * NVIDIA blog's layer adds the shared expert's output to the routed sum), in
 * this order with float32 accumulation and no atomics:
 *   y[t] = sum_{j=0}^{k-1} topk_w[t, j] * expert_out[pair_to_row[t*k + j]] + shared_out[t]
 * expert_out [T*k][d] and shared_out [T][d] (NULL: no shared term) are bf16 on
 * the FP8 and MXFP4 paths and float32 on the float32 path, as is y [T][d]. Pairs whose
 * pair_to_row is outside [0, T*k) contribute nothing.
 */
moe_status_t moe_combine(const moe_shape_t* shape, const void* expert_out,
                         const int32_t* pair_to_row, const float* topk_w,
                         const void* shared_out, void* y, void* stream);

/*
 * The whole layer: router, permutation, grouped FFN over the routed experts
 * and the shared expert, combine. x [T][d] and y [T][d] in act_dtype. The FP8
 * codes of x (quantised paths) are the ones moe_route_topk writes; above 64
 * tokens the layer computes them in its scan launch instead of the logits
 * launch (moe_layer_forward_overlap keeps them in the logits launch).
 * topk_ids [T][k] and topk_w [T][k] receive the routing when non-NULL. Needs a
 * workspace of moe_layer_workspace_size() bytes, aligned to 256 bytes.
 */
moe_status_t moe_layer_forward(const moe_shape_t* shape, const moe_weights_t* weights,
                               const void* x, void* y, int32_t* topk_ids, float* topk_w,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_layer_forward with the shared expert overlapped with the routing, as the
 * NVIDIA blog runs it (section "Cutting transformer-layer time by 34%": the
 * shared expert's computation on a second stream, hidden behind the router
 * logits and top-k; Table 1 row "Shared expert compute"). The shared expert's
 * GEMMs go on side_stream, which waits for fork_event -- recorded on `stream`
 * right after the router's logits launch, which writes the FP8 x codes the
 * shared expert reads -- while `stream` runs the selection, the permutation
 * and the routed GEMMs; `stream` waits for join_event, recorded on side_stream
 * after the shared expert's down GEMM, before the combine. side_stream and
 * both events (hipStream_t, hipEvent_t; events created by the caller,
 * preferably without timing) belong to the caller and must be distinct; the
 * call enqueues work on both streams and returns. Results are bit-identical
 * to moe_layer_forward. Shapes without a shared expert, and the float32 path,
 * run entirely on `stream` (nothing is enqueued on side_stream). Workspace as
 * moe_layer_forward; a call must not overlap another call on the same
 * workspace or events.
 */
moe_status_t moe_layer_forward_overlap(const moe_shape_t* shape, const moe_weights_t* weights,
                                       const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       void* side_stream, void* fork_event, void* join_event);

/*
 * Where moe_layer_forward leaves its intermediate results inside its workspace:
 * byte offsets from the workspace start (MOE_NO_REGION where the shape has no
 * such result). They hold the results of the last call that used the
 * workspace once the stream has reached its end, until the next call:
 *   xq, x_scale        FP8 codes [T][d] and float32 scales [T] of x (quantised paths)
 *   offsets            int32 [E+1], sorted_pair and pair_to_row int32 [T*k]: the
 *                      permutation, as moe_permute defines it
 *   h, h_scale         the routed experts' SwiGLU output by grouped row: FP8 codes
 *                      [T*k][F] and float32 block scales [T*k][F/128] (float32
 *                      [T*k][F] and no scales on the float32 path)
 *   h_shared, h_shared_scale   the shared expert's, [T][F_shared] and [T][F_shared/128]
 *   expert_out         [T*k][d] by grouped row, shared_out [T][d] (bf16, or float32)
 * Host-only; nothing is enqueued.
 */
#define MOE_NO_REGION ((size_t)-1)
typedef struct moe_layer_regions {
  size_t xq, x_scale;
  size_t offsets, sorted_pair, pair_to_row;
  size_t h, h_scale, h_shared, h_shared_scale;
  size_t expert_out, shared_out;
} moe_layer_regions_t;

moe_status_t moe_layer_workspace_regions(const moe_shape_t* shape, moe_layer_regions_t* regions);

/* Steps of moe_layer_forward, in launch order (for moe_layer_forward_events). */
typedef enum moe_step {
  MOE_STEP_ROUTE = 0,    /* router: logits and top-k kernels (T <= 64: the logits launch
                            also quantises x, and the top-k kernel does the permutation and
                            writes the FFN tile lists) */
  MOE_STEP_PERMUTE = 1,  /* permutation: scan (which also writes the FFN tile lists and,
                            T > 64, quantises x beside its one scanning workgroup) and
                            scatter; no kernels when T <= 64 */
  MOE_STEP_TILES = 2,    /* separate FFN tile-list kernel (moe_grouped_ffn only; none in the layer) */
  MOE_STEP_GATE_UP = 3,  /* gate/up GEMM + SwiGLU + h quantisation */
  MOE_STEP_DOWN = 4,     /* down GEMM */
  MOE_STEP_COMBINE = 5,  /* combine */
  MOE_NUM_STEPS = 6
} moe_step_t;

/*
 * moe_layer_forward that also records caller-created HIP events (hipEvent_t)
 * on `stream`: start_events[i] just before the first kernel of step i and
 * stop_events[i] just after its last kernel. Either array, or any entry, may
 * be NULL to skip it. Results are identical to moe_layer_forward.
 */
moe_status_t moe_layer_forward_events(const moe_shape_t* shape, const moe_weights_t* weights,
                                      const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* start_events, void* const* stop_events);

/*
 * Host-side copy of the E4M3 encoder the kernels use (float32 -> code, round
 * to nearest even, saturating at +-448), for testing it without a GPU.
 */
void moe_host_e4m3_encode(const float* in, uint8_t* out, int64_t n);

/* ---- QK-Norm + RoPE ---------------------------------------------------------
 * The step before attention in the same transformer layer, which the NVIDIA
 * Sarvam blog runs as one fused in-place pass over the query and key heads
 * (Table 1, row "QK Norm + RoPE", and the paragraph on fused positional
 * embedding): instead of a norm pass and a rotary pass that each read and
 * write the heads, every head is read once, normalised, rotated and written
 * back in place.
 *
 * For every token t (position p = positions[t]) and every query head h (and
 * likewise every key head, with k_weight):
 *   n[i]  = x[i] / sqrt(mean_j x[j]^2 + eps) * q_weight[i]          (RMSNorm)
 *   pair (a, b) of n with pair index i in [0, head_dim/2) becomes
 *   (a cos f - b sin f, a sin f + b cos f),  f = p * theta^(-2i / head_dim)
 * where the pairs are (2i, 2i+1) (MOE_ROPE_INTERLEAVED, the rotary-embedding
 * paper's definition) or (i, i + head_dim/2) (MOE_ROPE_HALVES). Value heads
 * and every other column of a row are not touched. Arithmetic in float32, the
 * angles' sines and cosines in float64; bf16 results rounded to nearest even.
 *
 * Layout: qkv [T][row_stride] elements of `dtype`, query head h at columns
 * [q_offset + h head_dim, +head_dim), key head h at k_offset + h head_dim;
 * the query and key column ranges must lie within the row and not overlap.
 * positions [T] int32 (any value). q_weight, k_weight [head_dim] of `dtype`.
 * qkv, q_weight and k_weight must be 16-byte aligned, and row_stride,
 * q_offset and k_offset multiples of 16 bytes' worth of elements (8 bf16,
 * 4 float32). All pointers are device memory owned by the caller; the call
 * enqueues one kernel on `stream` and returns. T == 0 is a no-op.
 * Errors (before any launch): MOE_ERR_INVALID_ARG for a null or misaligned
 * pointer, head_dim not 64, 128 or 256, no heads or more than 256, ranges
 * outside the row or overlapping, negative or non-finite eps, non-positive or
 * non-finite theta, an unknown style; MOE_ERR_UNSUPPORTED for a dtype other
 * than bf16 or float32.
 */
typedef enum moe_rope_style {
  MOE_ROPE_INTERLEAVED = 0, /* pairs (2i, 2i+1) */
  MOE_ROPE_HALVES = 1       /* pairs (i, i + head_dim/2) */
} moe_rope_style_t;

typedef struct moe_qk_shape {
  int32_t T;          /* tokens (rows of qkv), 0 <= T <= MOE_MAX_T */
  int32_t n_q;        /* query heads */
  int32_t n_kv;       /* key heads; 1 <= n_q + n_kv <= 256 */
  int32_t head_dim;   /* 64, 128 or 256 */
  int64_t row_stride; /* elements from one token's row to the next */
  int64_t q_offset;   /* element offset of query head 0 within a row */
  int64_t k_offset;   /* element offset of key head 0 within a row */
  float eps;          /* RMSNorm epsilon, inside the square root */
  float theta;        /* rotary base */
  int32_t style;      /* moe_rope_style_t */
  int32_t dtype;      /* MOE_DTYPE_BF16 or MOE_DTYPE_F32 (qkv and both weights) */
} moe_qk_shape_t;

moe_status_t moe_qk_norm_rope(const moe_qk_shape_t* shape, void* qkv, const int32_t* positions,
                              const void* q_weight, const void* k_weight, void* stream);

/* ---- the layer without a caller workspace -------------------------------------
 * For callers that cannot allocate device memory: code that a HIP graph
 * captures, tight serving loops, harnesses that forbid allocation. The same
 * computation and kernels as moe_layer_forward, bit-identical results, with
 * the workspace in a static device array of the library of
 * MOE_NOALLOC_SCRATCH_BYTES bytes: 32 MiB holds the workspace of the 30B-shaped
 * layer (d = 4096, E = 128, top-6, F = F_shared = 1024) up to T = 434 tokens
 * (a decode step, or a 256-token prefill chunk with 32 decode tokens), and of
 * the 100B-shaped layer (top-8, F = 2048) up to T = 318. Each GPU the library runs on holds
 * its own copy from the first call on that GPU until the process ends; that
 * first call looks up the array's device address (make it before any graph
 * capture). The call allocates nothing, frees nothing and enqueues only
 * kernels. Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, or graphs replayed concurrently) race
 * and must be serialised by the caller. Nothing in the array needs to start at
 * zero; it keeps the last call's intermediate results (at the offsets
 * moe_layer_workspace_regions gives). Arguments as moe_layer_forward; a shape
 * whose workspace exceeds the array returns MOE_ERR_SCRATCH before anything is
 * enqueued.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

moe_status_t moe_layer_forward_noalloc(const moe_shape_t* shape, const moe_weights_t* weights,
                                       const void* x, void* y, int32_t* topk_ids, float* topk_w,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
