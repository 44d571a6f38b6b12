"""Pins for the oracle's scalar numerics (bf16 encode/decode, GELU, SiLU)."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, f64_to_bf16_bits, gelu_erf, silu


def test_bf16_decode_ieee_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x0080], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 2.0 ** -126]
    got = bf16_to_f64(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e37).astype(np.float32),    # near overflow
        np.array([3.3961e38, -3.3961e38, 3.4e38], dtype=np.float32),
    ])
    # exact ties: lower 16 bits == 0x8000, both parities of the kept half
    u = rng.integers(0x00800000, 0x7F000000, 20000, dtype=np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(f64_to_bf16_bits(x.astype(np.float64)), _torch_bf16_bits(x))


def test_bf16_encode_single_rounding_from_f64():
    one = 1.0
    cases = {
        one + 2.0 ** -8 + 2.0 ** -40: 0x3F81,   # just above the tie: rounds up
        one + 2.0 ** -8: 0x3F80,                # exact tie, even neighbour is 1.0
        one + 3 * 2.0 ** -8: 0x3F82,            # exact tie, even neighbour is 1 + 2^-6
        one + 2.0 ** -8 - 2.0 ** -40: 0x3F80,   # just below the tie
        -(one + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -134: 0x0000,                    # half the smallest subnormal, tie to even (0)
        3 * 2.0 ** -134: 0x0002,                # 1.5 quanta: tie, to even (2 quanta)
    }
    for v, b in cases.items():
        assert int(f64_to_bf16_bits(np.array([v]))[0]) == b, v
    assert int(f64_to_bf16_bits(np.array([np.nan]))[0]) == 0x7FC0
    assert int(f64_to_bf16_bits(np.array([1e300]))[0]) == 0x7F80


def test_gelu_closed_forms():
    assert gelu_erf(np.array([0.0]))[0] == 0.0
    # GELU(1) = Phi(1), the standard normal CDF at 1.
    assert abs(gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    # GELU(-1) = -(1 - Phi(1))
    assert abs(gelu_erf(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15
    x = np.linspace(-8, 8, 4001)
    # GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1)
    assert np.max(np.abs(gelu_erf(x) - gelu_erf(-x) - x)) < 1e-14
    # asymptotes
    assert abs(gelu_erf(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(gelu_erf(np.array([-40.0]))[0]) < 1e-12
    # the tanh approximation stays within 5e-4 of the exact form (sanity on scale)
    tanh_form = 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))
    assert np.max(np.abs(tanh_form - gelu_erf(x))) < 5e-4


def test_silu_closed_forms():
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    x = np.linspace(-30, 30, 6001)
    assert np.max(np.abs(silu(x) - silu(-x) - x)) < 1e-13
    assert abs(silu(np.array([-800.0]))[0]) < 1e-300
    assert silu(np.array([800.0]))[0] == 800.0
    # sigma(x) = 1/(1+e^-x) evaluated one value at a time with math.exp
    for v in [-5.5, -0.25, 0.3, 2.0, 9.0]:
        assert abs(silu(np.array([v]))[0] - v / (1 + math.exp(-v))) < 1e-15
