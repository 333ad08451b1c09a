"""Seeded synthetic inputs for the QK-Norm + RoPE step (random numbers only;
none of the step's arithmetic).

Layout: one row per token of the fused QKV projection output, [T][row] with
row = (n_q + 2 n_kv) * head_dim + pad: query heads first, then key heads,
then value heads, then `pad` columns that must come back unchanged.

Distributions (the pages give none): q, k, v ~ N(0, 1); the two norm weights
~ N(1, 0.2^2); stored bf16 or float32. Positions: "prefill" 0..T-1 (one
request); "decode" each token a different request at 3584 + U[0, 128) (the
pages' input length plus a step of the output); "random" U[0, 2^20).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class QkConfig:
    name: str
    T: int
    n_q: int
    n_kv: int
    head_dim: int
    precision: str        # "bf16" or "f32"
    style: str            # "interleaved" or "halves"
    pos_mode: str         # "prefill", "decode" or "random"
    seed: int
    pad: int = 0
    theta: float = 10000.0
    eps: float = 1e-6

    @property
    def row(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim + self.pad

    @property
    def q_offset(self) -> int:
        return 0

    @property
    def k_offset(self) -> int:
        return self.n_q * self.head_dim

    def with_(self, **kw) -> "QkConfig":
        return replace(self, **kw)


# 30B-shaped attention heads (32 query, 4 key/value heads of 128): the page's
# listing compresses keys and values 8:1 against the model width 4096.
QK_CONFIGS = {
    "qk_prefill": QkConfig("qk_prefill", 3584, 32, 4, 128, "bf16", "halves", "prefill", seed=40),
    "qk_decode": QkConfig("qk_decode", 64, 32, 4, 128, "bf16", "halves", "decode", seed=41),
}

QK_PARITY = {
    "qk_small": QkConfig("qk_small", 37, 4, 2, 64, "bf16", "interleaved", "random", seed=42),
    "qk_small_halves": QkConfig("qk_small_halves", 37, 4, 2, 64, "bf16", "halves", "random", seed=43),
    "qk_f32_pad": QkConfig("qk_f32_pad", 19, 6, 2, 128, "f32", "halves", "random", seed=44, pad=12),
    "qk_f32_interleaved": QkConfig("qk_f32_interleaved", 11, 3, 1, 256, "f32", "interleaved",
                                   "prefill", seed=45, theta=500000.0),
    "qk_hd256": QkConfig("qk_hd256", 9, 2, 1, 256, "bf16", "halves", "random", seed=46, pad=8),
    "qk_one": QkConfig("qk_one", 1, 1, 1, 128, "bf16", "interleaved", "decode", seed=47, eps=0.5),
    "qk_many_heads": QkConfig("qk_many_heads", 5, 96, 16, 128, "bf16", "halves", "random", seed=48),
    # fewer 16-byte chunks per token than the sin/cos table has pairs
    "qk_hd256_two_heads": QkConfig("qk_hd256_two_heads", 3, 1, 1, 256, "bf16", "interleaved",
                                   "random", seed=49),
    # a large odd token count
    "qk_two_per_block_tail": QkConfig("qk_two_per_block_tail", 1025, 8, 2, 64, "bf16", "halves",
                                      "prefill", seed=50),
    # 3 heads of 16 lanes: the wave's last 16 lanes hold no chunk but hold the
    # cos/sin of pairs 48..63
    "qk_idle_lanes": QkConfig("qk_idle_lanes", 7, 2, 1, 128, "bf16", "halves", "random", seed=51),
    "qk_idle_lanes_f32": QkConfig("qk_idle_lanes_f32", 7, 1, 0, 256, "f32", "interleaved",
                                  "random", seed=52, pad=4),
    # over a thousand tokens of float32 heads, an odd count
    "qk_many_tail_f32": QkConfig("qk_many_tail_f32", 1030, 4, 2, 128, "f32", "interleaved",
                                 "prefill", seed=54),
    # 2048 chunks per token: two passes of 1024 threads
    "qk_two_passes": QkConfig("qk_two_passes", 3, 120, 8, 128, "bf16", "interleaved", "decode",
                              seed=53),
}


def qk_get(name: str) -> QkConfig:
    return QK_CONFIGS[name] if name in QK_CONFIGS else QK_PARITY[name]


@dataclass
class QkTensors:
    cfg: QkConfig
    qkv: torch.Tensor        # [T][row], bf16 or float32
    positions: torch.Tensor  # [T] int32
    q_weight: torch.Tensor   # [head_dim]
    k_weight: torch.Tensor   # [head_dim]


def _store(a: np.ndarray, precision: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if precision == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


def make_qk(cfg: QkConfig, device="cpu") -> QkTensors:
    ss = np.random.SeedSequence(cfg.seed).spawn(3)
    rx, rw, rp = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    qkv = rx.standard_normal((cfg.T, cfg.row), dtype=np.float32)
    w = 1.0 + 0.2 * rw.standard_normal((2, cfg.head_dim), dtype=np.float32)
    if cfg.pos_mode == "prefill":
        pos = np.arange(cfg.T)
    elif cfg.pos_mode == "decode":
        pos = 3584 + rp.integers(0, 128, cfg.T)
    elif cfg.pos_mode == "random":
        pos = rp.integers(0, 1 << 20, cfg.T)
    else:
        raise ValueError(cfg.pos_mode)
    return QkTensors(cfg, _store(qkv, cfg.precision, device),
                     torch.from_numpy(pos.astype(np.int32)).to(device),
                     _store(w[0], cfg.precision, device), _store(w[1], cfg.precision, device))


def values(t: torch.Tensor) -> np.ndarray:
    """Stored values as float64 numpy (exact for bf16 and float32)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
