"""Seeded synthetic input generators for the routed-expert-cache MoE layer.

This package produces *inputs only*: weights, activations, router logits,
sticky routing traces and the shapes of the five workloads.  It holds none of
the layer's arithmetic (no top-k, no cache policy, no FFN); both the CPU
oracle's tests and the HIP library's tests/benchmarks draw their inputs here.
"""
from .configs import CONFIGS, TinyCfg, DecodeBF16Cfg, DecodeFP8Cfg, PrefillBF16Cfg, PrefillFP8Cfg  # noqa: F401
from . import gen  # noqa: F401
