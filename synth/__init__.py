"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package only draws random numbers and encodes them as the byte layouts the
library consumes (bf16 bit patterns, fp32, int32).  It holds none of the
arithmetic of the method itself: no GEMM, no activation, no reduction and no
routing bookkeeping.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    ag_inputs,
    rs_inputs,
    mlp2_inputs,
    moe_inputs,
    zipf_probs,
)
