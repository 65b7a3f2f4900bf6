"""Row-major <-> MX_TILED conversions for test inputs and outputs (numpy).

MX_TILED (include/fp4dit.h): codes in 128-byte tiles of 2 rows x 128
elements, tile (r/2, k/128) at ((r/2)*(cols/128) + k/128)*128 with row r%2 at
+64*(r%2); scales in 128-byte tiles of 32 rows x 4 blocks, byte of (r, b) at
((r/32)*(cols/128) + b/4)*128 + (r%32)*4 + b%4.  Rows are padded (to 2 and
to 32); padding bytes are zero here and never read by the library.
"""

import numpy as np


def _round_up(v, m):
    return (v + m - 1) // m * m


def tile_codes(packed):
    """Row-major packed codes [rows, cols/2] -> tiled bytes [round_up(rows,2), cols/2]."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    rp = _round_up(rows, 2)
    p = np.zeros((rp, half), np.uint8)
    p[:rows] = packed
    return p.reshape(rp // 2, 2, half // 64, 64).transpose(0, 2, 1, 3).reshape(rp, half)


def untile_codes(tiled, rows, cols):
    t = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    rp = _round_up(rows, 2)
    t = t[: rp * cols // 2].reshape(rp // 2, cols // 128, 2, 64).transpose(0, 2, 1, 3).reshape(rp, cols // 2)
    return t[:rows]


def tile_scales(scales):
    """Row-major scales [rows, cols/32] -> tiled bytes [round_up(rows,32), cols/32]."""
    s = np.asarray(scales, dtype=np.uint8)
    rows, nb = s.shape
    rp = _round_up(rows, 32)
    p = np.zeros((rp, nb), np.uint8)
    p[:rows] = s
    return p.reshape(rp // 32, 32, nb // 4, 4).transpose(0, 2, 1, 3).reshape(rp, nb)


def untile_scales(tiled, rows, cols):
    t = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    rp = _round_up(rows, 32)
    nb = cols // 32
    t = t[: rp * nb].reshape(rp // 32, nb // 4, 32, 4).transpose(0, 2, 1, 3).reshape(rp, nb)
    return t[:rows]
