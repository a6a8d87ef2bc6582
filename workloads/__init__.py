"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package only draws random numbers and rounds them to the storage dtype. It
holds none of the attention method's arithmetic, so both the CPU oracle and the
GPU library can consume its tensors without sharing any code with each other.
"""

from .gaussian_mixture import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_head,
    make_inputs,
    scaled_config,
)
