"""Named layer shapes.

The five workloads follow the model shapes on the NVIDIA blog "How NVIDIA
extreme hardware-software co-design delivered a large inference boost for
Sarvam AI's sovereign models" (section "Scaling multilingual sovereign AI with
MoE": 128 routed experts, top-6 for the 30B model; top-8 and MoE FFN width
2048 for the 100B model; one shared expert) and its serving profile (section
"Performance challenges": input length 3584 tokens, 32-64 concurrent
requests). The hidden size 4096 and the 30B expert width 1024 are not on the
pages; they are this project's stated workload.

The remaining shapes are small parity cases: sizes the CPU oracle finishes in
seconds that still span several kernel tiles and leave ragged tails.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    d: int          # hidden size
    E: int          # routed experts
    k: int          # experts per token
    F: int          # routed expert FFN width
    F_shared: int   # shared expert FFN width (0: no shared expert)
    precision: str  # "fp8": bf16 activations + FP8 E4M3 weights; "mxfp4": bf16
                    # activations + OCP MXFP4 weights; "f32": float32 throughout
    seed: int
    skew: bool = False   # seeded per-expert router bias: 8 hot experts, 40 starved

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


CONFIGS = {
    # tiny float32 layer: T=16, d=256, E=8, top-2, F=128, one shared expert
    "tiny": LayerConfig("tiny", 16, 256, 8, 2, 128, 128, "f32", seed=1),
    # 30B-shaped decode step: 64 concurrent requests, one token each
    "decode": LayerConfig("decode", 64, 4096, 128, 6, 1024, 1024, "fp8", seed=2),
    # 30B-shaped prefill of one 3584-token request
    "prefill": LayerConfig("prefill", 3584, 4096, 128, 6, 1024, 1024, "fp8", seed=3),
    # 100B-shaped layer: top-8, FFN 2048, 4096 tokens
    "b100": LayerConfig("b100", 4096, 4096, 128, 8, 2048, 2048, "fp8", seed=4),
    # skewed routing: 8 hot experts take ~half the assignments, 40 get none
    "skew": LayerConfig("skew", 2048, 4096, 128, 6, 1024, 1024, "fp8", seed=5, skew=True),
    # a mixed batch: a 256-token prefill chunk and 32 decode tokens in one call
    "mixed": LayerConfig("mixed", 288, 4096, 128, 6, 1024, 1024, "fp8", seed=6),
    # the decode step and the prefill with MXFP4 expert weights
    "decode_mxfp4": LayerConfig("decode_mxfp4", 64, 4096, 128, 6, 1024, 1024, "mxfp4", seed=2),
    "prefill_mxfp4": LayerConfig("prefill_mxfp4", 3584, 4096, 128, 6, 1024, 1024, "mxfp4", seed=3),
}

# Small parity shapes (several tiles, ragged tails).
PARITY = {
    "f32_ragged": LayerConfig("f32_ragged", 37, 384, 12, 3, 256, 128, "f32", seed=11),
    "f32_noshared": LayerConfig("f32_noshared", 50, 256, 16, 4, 128, 0, "f32", seed=12),
    "fp8_small": LayerConfig("fp8_small", 45, 512, 16, 4, 256, 256, "fp8", seed=13),
    "fp8_ragged": LayerConfig("fp8_ragged", 203, 1024, 32, 6, 384, 256, "fp8", seed=14),
    "fp8_noshared": LayerConfig("fp8_noshared", 70, 512, 8, 2, 256, 0, "fp8", seed=15),
    "fp8_k1": LayerConfig("fp8_k1", 33, 256, 4, 1, 128, 128, "fp8", seed=16),
    "fp8_kE": LayerConfig("fp8_kE", 19, 256, 8, 8, 128, 128, "fp8", seed=17),
    "fp8_wide": LayerConfig("fp8_wide", 600, 2048, 64, 6, 512, 512, "fp8", seed=18),
    "fp8_skew_small": LayerConfig("fp8_skew_small", 512, 1024, 128, 6, 256, 256, "fp8",
                                  seed=19, skew=True),
    # the largest expert count: two 128-expert router tiles, a ragged token tail
    "fp8_e256": LayerConfig("fp8_e256", 130, 512, 256, 8, 128, 128, "fp8", seed=25),
    # two expert tiles in the tall-batch router at d = 1024, a ragged token tail
    "fp8_e256_rows": LayerConfig("fp8_e256_rows", 150, 1024, 256, 8, 128, 128, "fp8", seed=27),
    # one-tile batches (routing and permutation in one launch) with 4 and 3
    # experts per lane of the work-list wave, the 192-expert one ragged in T
    "fp8_e256_one_tile": LayerConfig("fp8_e256_one_tile", 64, 512, 256, 8, 128, 128, "fp8",
                                     seed=28),
    "fp8_e192_one_tile": LayerConfig("fp8_e192_one_tile", 41, 512, 192, 6, 256, 128, "fp8",
                                     seed=29),
    # the model's d = 4096 and F = 1024 (the shapes with fully unrolled K
    # loops) at few tokens, one per GEMM tile height: ~12, 24, 100 and 190
    # rows per expert select 16-, 32-, 128- and 192-row tiles
    "fp8_model_m16": LayerConfig("fp8_model_m16", 48, 4096, 16, 4, 1024, 1024, "fp8", seed=20),
    "fp8_model_m32": LayerConfig("fp8_model_m32", 96, 4096, 16, 4, 1024, 1024, "fp8", seed=21),
    "fp8_model_m128": LayerConfig("fp8_model_m128", 400, 4096, 8, 2, 1024, 1024, "fp8", seed=22),
    "fp8_model_m192": LayerConfig("fp8_model_m192", 380, 4096, 8, 4, 1024, 1024, "fp8", seed=23),
    # the 100B-shaped expert width F = 2048 (16 down K steps) with 128-row tiles
    "fp8_model_f2048": LayerConfig("fp8_model_f2048", 400, 4096, 8, 2, 2048, 2048, "fp8", seed=24),
    # ~150 rows per expert at F = 1024 select 192-row tiles and the tall down
    # GEMM; d = 640 leaves its last 256-channel N tile half outside d
    "fp8_tall_dpart": LayerConfig("fp8_tall_dpart", 600, 640, 8, 2, 1024, 1024, "fp8", seed=26),
    # MXFP4 expert weights (FP8 activations): small and model-shaped
    "mx_small": LayerConfig("mx_small", 45, 512, 16, 4, 256, 256, "mxfp4", seed=31),
    "mx_ragged": LayerConfig("mx_ragged", 203, 1024, 32, 6, 384, 256, "mxfp4", seed=32),
    "mx_model_m16": LayerConfig("mx_model_m16", 48, 4096, 16, 4, 1024, 1024, "mxfp4", seed=33),
    "mx_model_m64": LayerConfig("mx_model_m64", 200, 4096, 8, 2, 1024, 1024, "mxfp4", seed=34),
    "mx_model_m192": LayerConfig("mx_model_m192", 380, 4096, 8, 4, 1024, 1024, "mxfp4", seed=35),
    "mx_model_m128": LayerConfig("mx_model_m128", 400, 4096, 8, 2, 1024, 1024, "mxfp4", seed=39),
    "mx_model_m32": LayerConfig("mx_model_m32", 96, 4096, 16, 4, 1024, 1024, "mxfp4", seed=36),
    "mx_model_f2048": LayerConfig("mx_model_f2048", 400, 4096, 8, 2, 2048, 2048, "mxfp4", seed=37),
    "mx_tall_dpart": LayerConfig("mx_tall_dpart", 600, 640, 8, 2, 1024, 1024, "mxfp4", seed=38),
}


def get(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    return PARITY[name]
