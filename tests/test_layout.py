"""The test-side layout conversions match the address formulas of the C ABI."""

import numpy as np

import layout


def test_tiled_code_addresses():
    rng = np.random.default_rng(0)
    rows, cols = 5, 256
    packed = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    flat = layout.tile_codes(packed).reshape(-1)
    assert flat.size == 6 * cols // 2                  # padded to an even row count
    for r in range(rows):
        for k in range(0, cols, 2):
            off = ((r // 2) * (cols // 128) + k // 128) * 128 + (r % 2) * 64 + (k % 128) // 2
            assert flat[off] == packed[r, k // 2]
    assert np.array_equal(layout.untile_codes(flat, rows, cols), packed)


def test_tiled_scale_addresses():
    rng = np.random.default_rng(1)
    rows, cols = 40, 512
    s = rng.integers(0, 256, (rows, cols // 32)).astype(np.uint8)
    flat = layout.tile_scales(s).reshape(-1)
    assert flat.size == 64 * cols // 32                # padded to 32-row tiles
    for r in range(rows):
        for b in range(cols // 32):
            off = ((r // 32) * (cols // 128) + b // 4) * 128 + (r % 32) * 4 + b % 4
            assert flat[off] == s[r, b]
    assert np.array_equal(layout.untile_scales(flat, rows, cols), s)
