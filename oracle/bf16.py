"""Exact decoding of bfloat16 bit patterns for the oracle (test
infrastructure; see ``oracle/__init__.py``).

A bfloat16 value is the upper half of an IEEE float32, so widening the
16-bit pattern by 16 zero bits gives the float32 with the identical value;
the float64 of that is exact as well."""

import numpy as np


def bf16_bits_to_f64(bits):
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
