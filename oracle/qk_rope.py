"""QK-Norm + RoPE in float64: the step before attention that the NVIDIA Sarvam
blog fuses into one in-place pass over the query and key heads (Table 1, row
"QK Norm + RoPE", and the paragraph on fused positional embedding that
follows it).

TEST INFRASTRUCTURE (see the package docstring): used by the CPU pins, the GPU
parity tests and the benchmark's CPU-baseline leg only.

What it computes, for every token t and every query head and key head h (the
value heads and any other columns of the row are left as they are):

  1. RMSNorm over the head's head_dim values with a learned weight w (one
     weight vector for all query heads, another for all key heads):
        n[i] = x[i] / sqrt(mean_j x[j]^2 + eps) * w[i]
  2. Rotary position embedding at the token's position p: pair (a, b) of the
     head, pair index i in [0, head_dim/2), is rotated by the angle
     p * theta^(-2i / head_dim):
        a' = a cos - b sin,   b' = a sin + b cos.
     "interleaved" pairs elements (2i, 2i+1) as in the rotary-embedding
     paper's definition; "halves" pairs (i, i + head_dim/2).

Readings where the pages are silent (the blog names the fused step and its
time, nothing of its arithmetic): the norm is RMSNorm per head with eps inside
the square root; the norm comes before the rotation; the rotary base theta and
eps are parameters; both pairings are supported. All sums here are float64.
"""
from __future__ import annotations

import numpy as np

STYLES = ("interleaved", "halves")


def rms_norm_heads(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [..., head_dim], w [head_dim]: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """[T][head_dim/2]: position times theta^(-2i/head_dim)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    return np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]


def pair_views(head_dim: int, style: str):
    """Index arrays (first, second) of the rotated pairs within a head."""
    if style == "interleaved":
        return np.arange(0, head_dim, 2), np.arange(1, head_dim, 2)
    if style == "halves":
        h = head_dim // 2
        return np.arange(h), np.arange(h, head_dim)
    raise ValueError(style)


def rope(x: np.ndarray, positions: np.ndarray, theta: float, style: str) -> np.ndarray:
    """x [T][H][head_dim] rotated per token position."""
    x = np.asarray(x, np.float64)
    hd = x.shape[-1]
    ang = rope_angles(positions, hd, theta)[:, None, :]      # [T][1][hd/2]
    c, s = np.cos(ang), np.sin(ang)
    ia, ib = pair_views(hd, style)
    a, b = x[..., ia], x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = a * c - b * s
    out[..., ib] = a * s + b * c
    return out


def qk_norm_rope(qkv: np.ndarray, positions: np.ndarray, q_weight: np.ndarray,
                 k_weight: np.ndarray, n_q: int, n_kv: int, head_dim: int, q_offset: int,
                 k_offset: int, eps: float, theta: float, style: str) -> np.ndarray:
    """qkv [T][row] values (float64); q heads at columns q_offset + h*head_dim,
    key heads at k_offset + h*head_dim. Returns a new array with the query and
    key heads normalised and rotated, every other column unchanged."""
    out = np.array(qkv, dtype=np.float64, copy=True)
    T = out.shape[0]
    for off, nh, w in ((q_offset, n_q, q_weight), (k_offset, n_kv, k_weight)):
        cols = slice(off, off + nh * head_dim)
        heads = out[:, cols].reshape(T, nh, head_dim)
        out[:, cols] = rope(rms_norm_heads(heads, w, eps), positions, theta, style).reshape(T, -1)
    return out


def normalised_pairs(qkv: np.ndarray, q_weight, k_weight, n_q, n_kv, head_dim, q_offset,
                     k_offset, eps, style) -> np.ndarray:
    """|a| + |b| of each element's rotation pair after the norm, laid out like
    qkv (zero elsewhere): the scale of the float32 rounding error of a rotated
    element, for error bounds."""
    out = np.zeros(np.shape(qkv), dtype=np.float64)
    T = out.shape[0]
    ia, ib = pair_views(head_dim, style)
    for off, nh, w in ((q_offset, n_q, q_weight), (k_offset, n_kv, k_weight)):
        cols = slice(off, off + nh * head_dim)
        n = rms_norm_heads(np.asarray(qkv, np.float64)[:, cols].reshape(T, nh, head_dim), w, eps)
        m = np.abs(n[..., ia]) + np.abs(n[..., ib])
        sc = np.empty_like(n)
        sc[..., ia] = m
        sc[..., ib] = m
        out[:, cols] = sc.reshape(T, -1)
    return out
