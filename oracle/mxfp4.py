"""MXFP4 encoding: e2m1 elements with one e8m0 scale per 32 elements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources and readings
--------------------
* fal / Ideogram v4 page, section "Running the transformer in FP4": an FP4
  value has 1 sign bit, 2 exponent bits and 1 mantissa bit, so it takes one of
  a few levels.  Reading: exponent bias 1, exponent field 0 is subnormal, which
  gives the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* KroQuant summary, section "Deep analysis": the W4A4 format is MXFP4 (the
  page's bit description of it is garbled; it is read as e2m1 elements sharing
  one power-of-two scale per 32-element block).
* The page does not say how the block scale is chosen.  Reading (the OCP MX
  rule): shared exponent = floor(log2(amax)) - 2, where 2 is the largest
  e2m1 exponent, clamped to [-127, 127]; an all-zero block gets scale code 0.
  Elements are rounded to the nearest e2m1 level, ties to the level whose
  mantissa bit is 0 (round-to-nearest-even), magnitudes above 6 saturate to 6,
  and the sign bit is copied from the input (so -0 and small negatives give
  code 0b1000).
* Layout reading: blocks run along the last axis (K); codes are packed two per
  byte with the even element in the low nibble; scales are one byte per block,
  row-major [rows, cols/32].
"""

import math

import numpy as np

BLOCK = 32            # elements sharing one e8m0 scale
E2M1_EMAX = 2         # largest unbiased exponent of an e2m1 value (4 and 6)
E8M0_BIAS = 127


# ---------------------------------------------------------------- O1: e2m1 --
def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code: code = sign<<3 | exponent<<1 | mantissa.

    Exponent field 0 is subnormal (value = m * 0.5); otherwise the value is
    2**(e - 1) * (1 + m/2) (bias 1).
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAGNITUDES = E2M1_VALUES[:8]                      # codes 0..7, increasing
# Midpoint i lies between magnitude codes i and i+1.
E2M1_MIDPOINTS = 0.5 * (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:])


# ---------------------------------------------------------------- O2: e8m0 --
def e8m0_value(code):
    """Value of an e8m0 scale byte: 2**(code - 127); 255 is NaN."""
    code = np.asarray(code, dtype=np.int64)
    out = np.ldexp(1.0, code - E8M0_BIAS)
    return np.where(code == 255, np.nan, out)


# --------------------------------------------------------- O3: block scale --
def shared_exponent(amax):
    """Shared (unbiased) block exponent from the block's largest magnitude.

    floor(log2(amax)) is taken exactly from frexp (never from log2), minus the
    largest e2m1 exponent, clamped to the e8m0 range.  amax == 0 gives -127
    (scale code 0).  Vectorised over any array of amax values (float64).
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                      # amax = f * 2**e, f in [0.5, 1)
    floor_log2 = e.astype(np.int64) - 1
    shared = np.clip(floor_log2 - E2M1_EMAX, -127, 127)
    return np.where(amax == 0.0, -127, shared)


# ------------------------------------------------------ O4: element encode --
def encode_magnitude(q):
    """e2m1 magnitude code (0..7) of scaled magnitudes q >= 0 (float64).

    Nearest level; on an exact tie between two neighbouring levels the one
    with an even code (mantissa bit 0) wins; q beyond 6 saturates to code 7.
    Written as "count the midpoints below q", where a midpoint that q sits on
    exactly counts only if the code above it is even.
    """
    q = np.asarray(q, dtype=np.float64)
    code = np.zeros(q.shape, dtype=np.int64)
    for i, mid in enumerate(E2M1_MIDPOINTS):
        upper = i + 1
        passed = q > mid
        if upper % 2 == 0:
            passed = passed | (q == mid)
        code += passed
    return code


def quantize(x, return_scaled=False):
    """Quantise the rows of x (float64 values of fp32/bf16 inputs) to MXFP4.

    x: [rows, cols] with cols % 32 == 0.
    Returns (codes, scales): codes uint8 [rows, cols] (one 4-bit code per
    element, unpacked) and scales uint8 [rows, cols/32] (e8m0).  With
    return_scaled, also returns the exact scaled values x / 2**shared, used by
    the tests to tell genuine mismatches from rounding-order ties.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    # Step 1: amax per block (exact: abs and max do not round).
    amax = np.max(np.abs(xb), axis=2)
    # Step 2: shared exponent and its e8m0 code.
    shared = shared_exponent(amax)
    scales = (shared + E8M0_BIAS).astype(np.uint8)
    # Step 3: scale every element by 2**-shared (exact in float64).
    q = np.ldexp(xb, -shared[:, :, None])
    # Step 4: nearest e2m1 magnitude, sign bit copied from the input.
    mag = encode_magnitude(np.abs(q))
    sign = np.signbit(xb).astype(np.int64)
    codes = (sign << 3 | mag).astype(np.uint8).reshape(rows, cols)
    if return_scaled:
        return codes, scales, q.reshape(rows, cols)
    return codes, scales


# ---------------------------------------------------------- O5: dequantise --
def dequantize(codes, scales):
    """Exact float64 values of unpacked codes [rows, cols] with e8m0 scales."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, cols = codes.shape
    vals = E2M1_VALUES[codes].reshape(rows, cols // BLOCK, BLOCK)
    scale = e8m0_value(scales)[:, :, None]
    return (vals * scale).reshape(rows, cols)


# -------------------------------------------------------------- packing --
def pack_codes(codes):
    """Two codes per byte: element 2j in the low nibble, 2j+1 in the high."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """Inverse of pack_codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    out = np.empty((rows, 2 * half), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def floor_log2(v: float) -> int:
    """Exact floor(log2(v)) of a positive float, for scalar callers."""
    return math.frexp(v)[1] - 1
