"""Scalar numerics of the oracle: bf16 decoding/encoding and the two
activations used between the GEMMs.

bf16 is the operand type of every GEMM here: 1 sign bit, 8 exponent bits, 7
stored mantissa bits, i.e. the upper half of an IEEE binary32.  Encoding rounds
a float64 value once, to the nearest bf16, ties to the even significand.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf, expit as _expit


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even), return the bits.

    Normal range: |x| = m * 2^e with 0.5 <= m < 1 has 8 significant bits in
    bf16, so its quantum is 2^(e-8); below 2^-126 the quantum is fixed at
    2^-133 (bf16 subnormals).  Values that round beyond the largest finite
    bf16 become infinities; NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)
    u = f.view(np.uint32)
    out = (u >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out


def gelu_erf(x) -> np.ndarray:
    """GELU in its exact form, x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt 2)).

    The pages name a GeLU activation between the MLP's two GEMMs (TileLink,
    section 7.2) without fixing the form; the erf form is the definition."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def silu(x) -> np.ndarray:
    """SiLU, x * sigma(x) with sigma(x) = 1 / (1 + e^-x) (TileLink, section 7.2
    names SiLU-type activations between the FFN's two parts)."""
    x = np.asarray(x, dtype=np.float64)
    return x * _expit(x)
