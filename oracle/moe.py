"""CPU oracle for one mixture-of-experts layer forward pass (softmax top-k gating,
SwiGLU experts, one always-on shared expert).

TEST INFRASTRUCTURE. This module is the reference the HIP library is checked
against. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the library never does, and the two share no code.

Everything is float64 numpy, step by step in the order the method states, with
no blocking or fusion: a reader should be able to check each function against
its definition by eye. Where a decision turns a float into an integer (an FP8
code), it is taken in float32, the precision the GPU takes it in.

Sources (all on the web pages this project follows):
  * NVIDIA blog "How NVIDIA extreme hardware-software co-design delivered a
    large inference boost for Sarvam AI's sovereign models":
      - section "Scaling multilingual sovereign AI with MoE": 128 routed
        experts with top-6 routing (30B) and top-8 with MoE FFN width 2048
        (100B); a shared-expert design beside the routed experts;
      - Table 1 and the paragraph on MoE routing: router logits and top-k
        selection are one fused step; the routed experts run as grouped GEMMs;
        the shared expert is a separate computation that may overlap routing.
  * peacm.com repost, section 2.1: expert weights in FP8 (one byte per
    parameter); section 3.1: the fused router returns integer expert indices
    and float scores.
  * ijyty.com "InferX" page, section 2.4: softmax over the raw expert logits,
    then top-k; section 3.3: the router yields {indices: i32[k], weights:
    f32[k]} consumed by a fused scatter.

Readings where the pages are silent (each one is listed with its reason in the
design notes):
  R1 gate: softmax over all E logits (plus an optional per-expert bias), keep
     the k largest, renormalise their probabilities to sum to 1.
  R2 ties: order by logit descending, equal logits by lower expert index; ids
     are stored in that order.
  R3 permutation: pairs (t, j) grouped by expert, ascending token within a group.
  R4 SwiGLU: h = silu(gate) * up, silu(z) = z / (1 + exp(-z)); rows 0..F-1 of
     the stacked W13 are the gate projection, rows F..2F-1 the up projection.
  R5 shared expert: one, added with weight 1.
  R6 FP8 weights: OCP E4M3 codes with one float32 scale per output channel.
  R7 activations fed to FP8 GEMMs are themselves FP8: x per token, h per
     (row, 128-column block), each with a float32 scale amax/448 (1.0 when the
     amax is 0), codes by round-to-nearest-even with saturation.
  R8 output: bfloat16 (round to nearest even) on the FP8 path, float32 on the
     float32 path.
  R13 MXFP4 expert weights (a later format, the analogue of the NVFP4 weights
     the NVIDIA blog runs on Blackwell, section "Running on Blackwell"): OCP
     Microscaling MXFP4, E2M1 elements with one E8M0 power-of-two scale per 32
     along the reduction dimension and no channel scale; activations stay as
     in R7. A weight's value is its E2M1 value times its block's 2^(e - 127).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from . import codecs

H_BLOCK = 128  # width of one h-quantisation block (reading R7)


# ---------------------------------------------------------------------------
# Routing: router GEMM, softmax, top-k, renormalisation (NVIDIA blog, Table 1
# row "Router logits and TopK"; InferX page section 2.4).
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[e, i] (+ bias[e]); W_r is stored [E][d]."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the last axis (max subtracted first)."""
    z = l - l.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_ids(l: np.ndarray, k: int) -> np.ndarray:
    """The k expert indices per row, by logit descending, ties to the lower index.

    Top-k of the logits equals top-k of the softmax probabilities because
    softmax is strictly increasing in each logit.
    """
    T, E = l.shape
    out = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -l[t]))  # primary key: -l, secondary: index
        out[t] = order[:k]
    return out


def gate_weights(p: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, ids[t, j]] / sum_j' p[t, ids[t, j']] (renormalised top-k)."""
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k):
    """Routing of every token: (logits, probabilities, ids [T][k], weights [T][k])."""
    l = router_logits(x, w_router, bias)
    p = softmax(l)
    ids = topk_ids(l, k)
    w = gate_weights(p, ids)
    return l, p, ids, w


# ---------------------------------------------------------------------------
# Permutation of (token, slot) pairs into expert-contiguous order (the scatter
# the InferX page, section 3.3, fuses after the router).
# ---------------------------------------------------------------------------

@dataclass
class Permutation:
    counts: np.ndarray       # [E] rows per expert
    offsets: np.ndarray      # [E+1] first row of each expert's group
    sorted_pair: np.ndarray  # [T*k] row -> pair index t*k + j
    pair_to_row: np.ndarray  # [T*k] pair index -> row


def permute(ids: np.ndarray, E: int) -> Permutation:
    """Stable sort of the pairs p = t*k + j by expert id (reading R3).

    Stability keeps pairs of one expert in increasing p, hence increasing t
    (a token's k ids are distinct, so no two pairs of one group share a t).
    """
    flat = ids.reshape(-1).astype(np.int64)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_to_row = np.empty_like(sorted_pair)
    pair_to_row[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    return Permutation(counts, offsets, sorted_pair, pair_to_row)


def tile_histogram(ids: np.ndarray, E: int, tile: int = 64) -> np.ndarray:
    """counts[i][e] = number of tokens among rows [tile i, tile (i + 1)) of ids
    that chose expert e (the per-tile histogram a counting permutation starts
    from); ids outside [0, E) are not counted."""
    T = ids.shape[0]
    n = -(-T // tile)
    out = np.zeros((n, E), dtype=np.int32)
    for i in range(n):
        block = ids[i * tile:(i + 1) * tile].reshape(-1)
        valid = block[(block >= 0) & (block < E)].astype(np.int64)
        out[i] = np.bincount(valid, minlength=E)
    return out


def gather_rows(xq: np.ndarray, s_x: np.ndarray, perm: Permutation, k: int):
    """The row copy of the scatter (InferX page, section 3.3): grouped row r
    holds the activation row of the token of pair sorted_pair[r], with its
    scale. Returns (x_perm [T*k][d], x_perm_scale [T*k])."""
    tok = perm.sorted_pair.astype(np.int64) // k
    return xq[tok], s_x[tok]


# ---------------------------------------------------------------------------
# FP8 activation quantisation (reading R7): decisions taken in float32.
# ---------------------------------------------------------------------------

def quantize_rows_e4m3(v: np.ndarray):
    """Per-row scale s = fp32(amax)/448 in float32 (1.0 if amax == 0) and codes
    E4M3(fp32(v) / s), the division in float32. Returns (codes uint8, s float32)."""
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.abs(v32).max(axis=-1)
    s = (amax / np.float32(codecs.E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = codecs.e4m3_encode(v32 / s[..., None])  # float32 / float32 -> float32
    return q, s


def quantize_blocks_e4m3(h: np.ndarray, block: int = H_BLOCK):
    """Quantise each row of h per `block`-wide column block. Returns
    (codes [R][C] uint8, scales [R][C/block] float32)."""
    R, C = h.shape
    assert C % block == 0
    hb = np.asarray(h, np.float32).reshape(R, C // block, block)
    q, s = quantize_rows_e4m3(hb)
    return q.reshape(R, C), s


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# Expert FFNs (SwiGLU; reading R4).
# ---------------------------------------------------------------------------

@dataclass
class ExpertWeights:
    """One expert, as stored. fmt "fp8": w13/w2 are uint8 E4M3 codes with
    float32 per-output-channel scales. fmt "mxfp4": w13 [2F][d/2] / w2
    [d][F/2] packed E2M1 codes with E8M0 block scales [2F][d/32] / [d][F/32]
    (OCP MXFP4, no channel scale). Float32 path: float arrays, scales None."""
    w13: np.ndarray                  # [2F][d]
    w13_scale: Optional[np.ndarray]  # [2F]
    w2: np.ndarray                   # [d][F]
    w2_scale: Optional[np.ndarray]   # [d]
    fmt: str = "fp8"


def ffn_fp32(x: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """Float32 path: o = W2 (silu(W1 x) * (W3 x)), all sums in float64."""
    F = ew.w13.shape[0] // 2
    w13 = np.asarray(ew.w13, np.float64)
    gu = np.asarray(x, np.float64) @ w13.T
    h = silu(gu[:, :F]) * gu[:, F:]
    return h @ np.asarray(ew.w2, np.float64).T


def gate_up_fp8(xq: np.ndarray, s_x: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """gu[r, n] = s_x[r] * s_w13[n] * sum_i xq[r, i] q13[n, i] for rows whose x
    is already quantised (codes xq, per-row scales s_x); columns n < F are the
    gate, n >= F the up projection. The dot products of E4M3 values are exact
    in float64 (every partial sum is a multiple of 2^-18 below 2^31)."""
    xv = codecs.e4m3_decode(xq)                                # [R][d]
    if ew.fmt == "mxfp4":  # each weight is its E2M1 value times its block's 2^e
        gu = xv @ codecs.mxfp4_decode(ew.w13, ew.w13_scale).T   # [R][2F]
        return gu * np.asarray(s_x, np.float64)[:, None]
    gu = xv @ codecs.e4m3_decode(ew.w13).T                      # [R][2F]
    return gu * np.asarray(s_x, np.float64)[:, None] * np.asarray(ew.w13_scale, np.float64)[None, :]


def swiglu_h_fp8(xq: np.ndarray, s_x: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """h = silu(gate) * up, before h is quantised."""
    F = ew.w13.shape[0] // 2
    gu = gate_up_fp8(xq, s_x, ew)
    return silu(gu[:, :F]) * gu[:, F:]


def down_fp8(hq: np.ndarray, s_h: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """o[m] = s_w2[m] * sum_b s_h[b] * sum_{n in b} hq[n] q2[m, n] (FP8
    weights); with MXFP4 weights q2 is the decoded weight (element times its
    block's 2^e) and there is no s_w2."""
    F = hq.shape[1]
    hv = codecs.e4m3_decode(hq)                                 # [R][F]
    mx = ew.fmt == "mxfp4"
    q2 = codecs.mxfp4_decode(ew.w2, ew.w2_scale) if mx else codecs.e4m3_decode(ew.w2)  # [d][F]
    o = np.zeros((hq.shape[0], q2.shape[0]), dtype=np.float64)
    for b in range(F // H_BLOCK):
        cols = slice(b * H_BLOCK, (b + 1) * H_BLOCK)
        o += np.asarray(s_h[:, b], np.float64)[:, None] * (hv[:, cols] @ q2[:, cols].T)
    return o if mx else o * np.asarray(ew.w2_scale, np.float64)[None, :]


def ffn_fp8(xq: np.ndarray, s_x: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """FP8 path of one expert on rows with quantised x: SwiGLU h, its
    per-(row, 128-column block) quantisation, then the down projection."""
    h = swiglu_h_fp8(xq, s_x, ew)
    hq, s_h = quantize_blocks_e4m3(h)
    return down_fp8(hq, s_h, ew)


# ---------------------------------------------------------------------------
# Whole layer.
# ---------------------------------------------------------------------------

@dataclass
class LayerInputs:
    """Host copies of every input, as stored (bf16 as uint16 bits, FP8 as uint8
    codes). `expert(e)` returns routed expert e; `shared` is the shared expert
    or None. precision: "fp8" (bf16 activations, FP8 weights), "mxfp4" (bf16
    activations, MXFP4 weights) or "f32"."""
    precision: str
    x: np.ndarray             # [T][d] uint16 bf16 bits, or float32
    w_router: np.ndarray      # [E][d] uint16 bf16 bits, or float32
    router_bias: Optional[np.ndarray]  # [E] float32 or None
    k: int
    E: int
    expert: Callable[[int], ExpertWeights]
    shared: Optional[ExpertWeights]


def activations(inp: LayerInputs) -> np.ndarray:
    """x as float64 (bf16 bit patterns decoded exactly)."""
    if inp.precision != "f32":
        return codecs.bf16_decode(inp.x)
    return np.asarray(inp.x, np.float64)


def router_weight(inp: LayerInputs) -> np.ndarray:
    if inp.precision != "f32":
        return codecs.bf16_decode(inp.w_router)
    return np.asarray(inp.w_router, np.float64)


@dataclass
class LayerResult:
    ids: np.ndarray
    w: np.ndarray
    perm: Optional[Permutation]
    xq: Optional[np.ndarray]
    s_x: Optional[np.ndarray]
    expert_out: Optional[np.ndarray]  # [T*k][d] in grouped-row order
    shared_out: Optional[np.ndarray]  # [T][d]
    y64: np.ndarray                   # [T][d] float64, before output rounding
    y: np.ndarray                     # [T][d] rounded to the output format (as float64)


def combine(w: np.ndarray, o_pairs: np.ndarray, o_shared: Optional[np.ndarray]) -> np.ndarray:
    """y[t] = sum_j w[t, j] * o[t, j] + o_shared[t]; o_pairs is [T][k][d]."""
    y = np.einsum("tj,tjd->td", np.asarray(w, np.float64), o_pairs)
    if o_shared is not None:
        y = y + o_shared
    return y


def round_output(y64: np.ndarray, precision: str) -> np.ndarray:
    if precision != "f32":
        return codecs.bf16_round(y64)
    return y64.astype(np.float32).astype(np.float64)


def layer_forward(inp: LayerInputs, keep_intermediates: bool = True) -> LayerResult:
    """The whole layer on every token: route, permute, per-expert FFN on the
    grouped rows, shared expert on all rows, combine."""
    x = activations(inp)
    T, d = x.shape
    k, E = inp.k, inp.E
    _, _, ids, w = route(x, router_weight(inp), inp.router_bias, k)
    perm = permute(ids, E)
    xq = s_x = None
    if inp.precision != "f32":
        xq, s_x = quantize_rows_e4m3(x)
    expert_out = np.zeros((T * k, d), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(perm.offsets[e]), int(perm.offsets[e + 1])
        if r1 == r0:
            continue  # empty group: no rows, no work
        tok = perm.sorted_pair[r0:r1] // k
        ew = inp.expert(e)
        if inp.precision != "f32":
            expert_out[r0:r1] = ffn_fp8(xq[tok], s_x[tok], ew)
        else:
            expert_out[r0:r1] = ffn_fp32(x[tok], ew)
    shared_out = None
    if inp.shared is not None:
        shared_out = (ffn_fp8(xq, s_x, inp.shared) if inp.precision != "f32"
                      else ffn_fp32(x, inp.shared))
    o_pairs = expert_out[perm.pair_to_row].reshape(T, k, d)
    y64 = combine(w, o_pairs, shared_out)
    return LayerResult(ids, w, perm, xq, s_x,
                       expert_out if keep_intermediates else None,
                       shared_out if keep_intermediates else None,
                       y64, round_output(y64, inp.precision))


def layer_forward_tokens(inp: LayerInputs, tokens: np.ndarray):
    """The layer's output for a subset of tokens only (each token's output
    depends on its own row alone). Returns (ids, w, xq, s_x, y64, y) for the
    given tokens; used to check full-size runs on sampled rows."""
    x = activations(inp)[tokens]
    k = inp.k
    _, _, ids, w = route(x, router_weight(inp), inp.router_bias, k)
    xq = s_x = None
    if inp.precision != "f32":
        xq, s_x = quantize_rows_e4m3(x)
    T, d = x.shape
    o_pairs = np.zeros((T, k, d), dtype=np.float64)
    for e in np.unique(ids):
        ew = inp.expert(int(e))
        rows, slots = np.nonzero(ids == e)
        if inp.precision != "f32":
            o_pairs[rows, slots] = ffn_fp8(xq[rows], s_x[rows], ew)
        else:
            o_pairs[rows, slots] = ffn_fp32(x[rows], ew)
    shared_out = None
    if inp.shared is not None:
        shared_out = (ffn_fp8(xq, s_x, inp.shared) if inp.precision != "f32"
                      else ffn_fp32(x, inp.shared))
    y64 = combine(w, o_pairs, shared_out)
    return ids, w, xq, s_x, y64, round_output(y64, inp.precision)


def near_tie_rows(l: np.ndarray, k: int, min_gap: float) -> np.ndarray:
    """Rows whose k+1 largest logits (sorted) have an adjacent gap below
    min_gap: there the top-k set or its order could flip between float32 and
    float64 arithmetic. Returns a boolean mask over rows."""
    E = l.shape[1]
    m = min(k + 1, E)
    top = -np.sort(-l, axis=1)[:, :m]
    if m < 2:
        return np.zeros(l.shape[0], dtype=bool)
    gaps = top[:, :-1] - top[:, 1:]
    return (gaps < min_gap).any(axis=1)
