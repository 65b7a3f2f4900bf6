"""Block-local invertible transform on activations, inverse folded into W.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: KroQuant summary page, "Background and overview" (an invertible
linear transform smooths the activations and its inverse is applied to the
weights; it must run online every denoising step) and "Deep analysis" (the
activations are split into independent 32-element blocks, each transformed by
a learned matrix, so the transform becomes small-tile matrix-core GEMMs).

Readings: the convention is y_b = x_b @ T_b for the b-th 32-element slice
x_b of a row; T holds either one matrix shared by every block (n_t = 1) or
one per block (n_t = K/32); T is given as bfloat16 values (exact in float64).
Since X @ W = sum_b X_b W_b = sum_b (X_b T_b)(T_b^-1 W_b), the weight side
is W'_b = T_b^-1 @ W_b for the 32 rows of W that block b multiplies.
"""

import numpy as np

from . import mxfp4

BLOCK = 32


def _block_matrix(t, n_t, b):
    return t[0] if n_t == 1 else t[b]


def block_transform(x, t):
    """y[:, 32b:32b+32] = x[:, 32b:32b+32] @ T_b in float64."""
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    rows, cols = x.shape
    n_t = t.shape[0]
    nb = cols // BLOCK
    if cols % BLOCK or n_t not in (1, nb) or t.shape[1:] != (BLOCK, BLOCK):
        raise ValueError("bad transform shape")
    y = np.empty_like(x)
    for b in range(nb):
        sl = slice(BLOCK * b, BLOCK * (b + 1))
        y[:, sl] = x[:, sl] @ _block_matrix(t, n_t, b)
    return y


def transform_quantize(x, t, return_scaled=False):
    """Block transform followed by MXFP4 quantisation of the result."""
    return mxfp4.quantize(block_transform(x, t), return_scaled=return_scaled)


def fold_inverse(w, t):
    """Weight side: W'[32b:32b+32, :] = T_b^-1 @ W[32b:32b+32, :] (float64).

    w is the logical weight [K, N] of y = x @ w.
    """
    w = np.asarray(w, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    k = w.shape[0]
    n_t = t.shape[0]
    out = np.empty_like(w)
    for b in range(k // BLOCK):
        sl = slice(BLOCK * b, BLOCK * (b + 1))
        out[sl] = np.linalg.solve(_block_matrix(t, n_t, b), w[sl])
    return out
