"""Seeded synthetic inputs for the centroid-masked sparse LM head.

This package only draws random numbers and lays them out; it holds none of the
head's arithmetic (no dot products, no selection, no argmax).  Both the CPU
oracle's tests and the GPU path's tests and benchmark take their inputs from
here, so the two sides always see the same bytes.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    f32_to_bf16_bits,
    make_random,
    make_workload,
    zipf_sizes,
)
