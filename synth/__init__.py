"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package draws random numbers and builds weight sets of the shapes the Parameter
Golf submission cards describe.  It holds none of the quantizer's arithmetic: no
scale, code, clip, mask, average or export decision is computed here.
"""
from .weights import (  # noqa: F401
    key_of,
    uniform01,
    normal,
    gauss_f32,
    gauss_bf16,
    student_t3_f32,
    lognormal_f32,
    f32_to_bf16_bits,
    SynthTensor,
    config1,
    config1_batch,
    config2,
    config3_weights,
    config3_grads,
    config4,
    config5_base,
    config5_snapshot,
    config5_snapshots,
    stress_s1,
    stress_s2,
    stress_s4_weights,
)
