"""Pins of the oracle's exact bfloat16 decoding.

A bfloat16 pattern is sign (1 bit), exponent (8 bits, bias 127) and the top 7
fraction bits of an IEEE binary32; the expected values below are worked out
from that layout by hand, not by widening the pattern."""

import math

import numpy as np

import oracle

CASES = [
    (0x3F80, 1.0),                          # exponent 127, fraction 0
    (0xC000, -2.0),                         # sign, exponent 128
    (0x4049, 3.140625),                     # 2 * (1 + 73/128)
    (0x3E00, 0.125),                        # exponent 124
    (0x0001, 2.0 ** -133),                  # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),            # largest subnormal
    (0x0080, 2.0 ** -126),                  # smallest normal
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x0000, 0.0),
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def test_bf16_bits_to_f64_values():
    bits = np.array([b for b, _ in CASES], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for (b, want), v in zip(CASES, got.tolist()):
        assert v == want, hex(b)


def test_bf16_negative_zero_and_nan():
    got = oracle.bf16_bits_to_f64(np.array([0x8000, 0x7FC0, 0xFFC1], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) == -1.0
    assert np.isnan(got[1]) and np.isnan(got[2])


def test_bf16_signed_16_bit_input():
    """The decoder takes the 16 bits whatever the integer type holds them:
    an int16 view of 0xC000 is -16384."""
    got = oracle.bf16_bits_to_f64(np.array([-16384, 16256], dtype=np.int16))
    assert got.tolist() == [-2.0, 1.0]
