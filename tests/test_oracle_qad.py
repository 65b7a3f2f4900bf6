"""Pins of the QAD fake-quantisation oracle (CPU only)."""

import numpy as np
import pytest

import golden_io
from oracle import qad

BLOCKS = golden_io.mxfp4_blocks()


def _hand_values(codes_packed, scale):
    """Values of a hand-worked block from the hand-written code table."""
    table = {c: v for c, _, _, _, v in golden_io.e2m1_table()}
    codes = []
    for b in codes_packed:
        codes += [b & 0xF, b >> 4]
    return np.array([table[c] * 2.0 ** (scale - 127) for c in codes])


def _same_bits(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("blk", [b for b in BLOCKS if b[2] != 255], ids=[b[0] for b in BLOCKS if b[2] != 255])
def test_fake_quantize_hand_worked_blocks(blk):
    name, x, scale, codes = blk
    y = qad.fake_quantize(np.array([x]))
    assert _same_bits(y[0], _hand_values(codes, scale)), name


def test_fake_quantize_is_idempotent_and_odd():
    rng = np.random.default_rng(70)
    x = rng.standard_normal((16, 256)) * 2.0 ** rng.integers(-20, 20, (16, 1))
    x[:, rng.choice(256, 4, replace=False)] *= 30
    y = qad.fake_quantize(x)
    assert _same_bits(qad.fake_quantize(y), y)
    assert _same_bits(qad.fake_quantize(-x), -y)


def test_fake_quantize_keeps_grid_values():
    """Grid values times 2^s, with an element of magnitude 4 or 6 times 2^s
    in every block (so the block exponent is s), come back unchanged."""
    rng = np.random.default_rng(71)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(grid, (8, 128)) * rng.choice([-1.0, 1.0], (8, 128))
    x[:, ::32] = rng.choice([4.0, 6.0, -4.0, -6.0], (8, 4))
    x *= 2.0 ** rng.integers(-100, 100, (8, 1))
    assert _same_bits(qad.fake_quantize(x), x)


def test_ste_passes_the_gradient_unchanged():
    """Also where the forward saturates or rounds to zero."""
    rng = np.random.default_rng(72)
    g = rng.standard_normal((4, 64))
    out = qad.ste_backward(g)
    assert _same_bits(out, g) and out is not g
