"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package generates inputs only: normal draws from numpy's PCG64, a fan-in
scale, and the exact round-to-nearest-even encoding of float32 draws into
bfloat16 bit patterns.  It contains none of the arithmetic of the tensor-parallel
layer itself, so both the CPU oracle and the HIP path may consume what it makes.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .synth import (  # noqa: F401
    HostTensor,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    generate,
    output_gradient,
)
