"""Seeded synthetic workloads: input generators, the named configurations, and FLOP/byte accounting.

This package holds none of the attention method's arithmetic. The tests and the bench use it to build the
same inputs for the HIP path and for the float64 oracle; neither of those two imports the other.
"""
from .inputs import (  # noqa: F401
    TENSOR_IDS,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    normal_bf16_bits,
    normal_bf16_slab,
    normal_f32,
    mask_probe_inputs,
)
from .configs import CONFIGS, Config  # noqa: F401
