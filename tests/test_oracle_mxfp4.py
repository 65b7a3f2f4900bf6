"""Pins of the MXFP4 oracle (CPU only).

Each check ties the oracle to something other than itself: the hand-written
code table, hand-worked blocks, exact rational brute force over every finite
bfloat16 value, and properties the encoding must have.
"""

import math

import numpy as np
import pytest

import bruteforce
import golden_io
from oracle import mxfp4


def test_e2m1_table_matches_hand_table():
    rows = golden_io.e2m1_table()
    assert [r[0] for r in rows] == list(range(16))
    for code, s, e, m, v in rows:
        assert code == (s << 3 | e << 1 | m)
        got = mxfp4.e2m1_value(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v)
    assert np.array_equal(mxfp4.E2M1_VALUES, [r[4] for r in rows])


def test_grid_is_the_fp4_value_grid():
    grid = {0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0, 3.0, -3.0, 4.0, -4.0, 6.0, -6.0}
    assert set(mxfp4.E2M1_VALUES.tolist()) == grid
    assert list(mxfp4.E2M1_MAGNITUDES) == sorted(mxfp4.E2M1_MAGNITUDES)


def test_e8m0_values():
    assert mxfp4.e8m0_value(127) == 1.0
    assert mxfp4.e8m0_value(0) == 2.0 ** -127
    assert mxfp4.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(mxfp4.e8m0_value(255))


@pytest.mark.parametrize("block", golden_io.mxfp4_blocks(), ids=lambda b: b[0])
def test_hand_worked_blocks(block):
    name, x, scale, packed = block
    codes, scales = mxfp4.quantize(np.array([x]))
    assert int(scales[0, 0]) == scale
    assert mxfp4.pack_codes(codes)[0].tolist() == packed
    # the rational brute force agrees on the same hand-worked blocks
    bs, bc = bruteforce.encode_block(x)
    assert bs == scale and bc == codes[0].tolist()


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    return vals[np.isfinite(vals)].astype(np.float64)


def test_every_bf16_value_against_brute_force():
    """Every finite bf16 value x, in blocks whose largest magnitude is |x|
    itself or 2**d times the top of x's binade (d = 1..4), so that the scaled
    value sweeps every e2m1 interval, midpoint and the saturating range."""
    vals = _all_finite_bf16()
    blocks = []
    for x in vals:
        ax = abs(x)
        companions = [0.0]
        if ax != 0:
            top = 2.0 ** (math.frexp(ax)[1])           # next power of two above |x|
            companions += [top * 2.0 ** d for d in (0, 1, 2, 3)]
        for c in companions:
            if not math.isfinite(c):
                continue
            blocks.append([x, c] + [0.0] * 30)
    xs = np.array(blocks)
    codes, scales = mxfp4.quantize(xs)
    for i in range(len(xs)):
        s, c = bruteforce.encode_block(xs[i].tolist(), only=2)
        assert int(scales[i, 0]) == s, xs[i, :2]
        assert codes[i, :2].tolist() == c, xs[i, :2]
    # and structurally for every block: the zero padding encodes to code 0
    assert not codes[:, 2:].any()


def test_random_blocks_against_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(300):
        scale = 2.0 ** rng.integers(-140, 120)
        x = rng.standard_normal(32) * scale
        x[rng.integers(0, 32, 3)] *= 20.0                  # outliers
        x = x.astype(np.float32).astype(np.float64)
        codes, scales = mxfp4.quantize(x[None])
        s, c = bruteforce.encode_block(x.tolist())
        assert int(scales[0, 0]) == s
        assert codes[0].tolist() == c


def test_idempotent():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-20, 20, (64, 1)))
    c1, s1 = mxfp4.quantize(x)
    d = mxfp4.dequantize(c1, s1)
    c2, s2 = mxfp4.quantize(d)
    assert np.array_equal(s1, s2)
    # -0 dequantises to -0 and re-encodes to 0x8, so codes match exactly
    assert np.array_equal(c1, c2)


def test_monotone_within_block():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 32)) * 3
    codes, _ = mxfp4.quantize(x)
    mags = codes & 7
    order = np.argsort(np.abs(x), axis=1)
    sorted_mags = np.take_along_axis(mags, order, axis=1)
    assert (np.diff(sorted_mags.astype(int), axis=1) >= 0).all()


def test_error_bound():
    """|D(Q(x)) - x| <= half the local grid gap (times the scale) when the
    scaled value is inside the grid; beyond 6 the error is |q| - 6 < 2."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((500, 32)) * 2.0 ** rng.integers(-8, 8, (500, 1))
    codes, scales, q = mxfp4.quantize(x, return_scaled=True)
    d = mxfp4.dequantize(codes, scales)
    scale = np.repeat(mxfp4.e8m0_value(scales), 32, axis=1)
    aq = np.abs(q)
    gap = np.where(aq < 2, 0.5, np.where(aq < 4, 1.0, 2.0))
    inside = aq <= 6
    err = np.abs(d - x) / scale
    assert (err[inside] <= gap[inside] / 2 + 1e-12).all()
    assert (err[~inside] < 2).all()
    assert aq.max() < 8


def test_shared_exponent_edges():
    assert mxfp4.shared_exponent(0.0) == -127
    assert mxfp4.shared_exponent(4.0) == 0
    assert mxfp4.shared_exponent(7.999) == 0
    assert mxfp4.shared_exponent(8.0) == 1
    assert mxfp4.shared_exponent(2.0 ** -140) == -127
    assert mxfp4.shared_exponent(2.0 ** 127 * 1.5) == 125


def test_pack_roundtrip_and_order():
    codes = np.array([[1, 2, 3, 4, 15, 0, 8, 7]], dtype=np.uint8)
    packed = mxfp4.pack_codes(codes)
    assert packed.tolist() == [[0x21, 0x43, 0x0F, 0x78]]
    assert np.array_equal(mxfp4.unpack_codes(packed), codes)
