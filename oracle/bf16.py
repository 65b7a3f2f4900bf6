"""Round float64 values to bfloat16 (round-to-nearest-even) for output compares.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say nothing about how outputs are rounded; the reading taken is
round-to-nearest-even.  The value is first rounded to float32 (NumPy's cast is
RNE) and then to bfloat16 by rounding away the low 16 mantissa bits with ties
to even; the double rounding differs from a direct float64 -> bf16 rounding
only on values within 2**-24 relative of a bf16 midpoint, far inside the
output tolerance.
"""

import numpy as np


def to_bf16_bits(x):
    """uint16 bfloat16 bit patterns of float64 values (NaN kept as NaN)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(f)
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def from_bf16_bits(b):
    """float64 values of uint16 bfloat16 bit patterns (exact)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """float64 -> nearest bfloat16 value, returned as float64."""
    return from_bf16_bits(to_bf16_bits(x))
