"""Seeded synthetic workloads for the MoE layer (shapes and input generator).

Shared by the tests, the benchmark and the smoke check. Holds no arithmetic of
the layer itself; see `gen.py` for the distributions.
"""
from .configs import CONFIGS, PARITY, LayerConfig, get  # noqa: F401
from .gen import LayerTensors, make_layer, act_values  # noqa: F401
