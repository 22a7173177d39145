"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This package holds input *formats and recipes only*: random draws, rounding to
16-bit storage formats, and the structure of each workload (shapes, spikes,
sampled rows). It contains none of the attention arithmetic.
"""
from .inputs import (  # noqa: F401
    FMT_F16,
    FMT_BF16,
    f32_to_bits,
    bits_to_f64,
    bits_to_f32,
    normal_bits,
    Workload,
    tiny_fwd,
    a100_sweep,
    spiked_causal,
    long_causal,
    fwd_bwd,
    random_case,
    long_causal_sample_rows,
)
