"""Seeded synthetic inputs for the selected-key / split-K attention workloads.

This package only draws numbers and lays them out in storage formats (fp32,
fp16, bf16 bit patterns, int8 rows with a per-row fp32 scale). It holds none of
the attention arithmetic, so both the FP64 oracle and the HIP path can consume
its arrays without sharing any computation.
"""

from .gen import (  # noqa: F401
    DecodeWorkload,
    PrefillWorkload,
    f32_to_bf16_bits,
    quantize_rows_i8,
    make_decode,
    make_prefill_mask,
    make_prefill_sel,
    config1,
    config2,
    config3,
    config4,
    config5,
    CONFIGS,
)
