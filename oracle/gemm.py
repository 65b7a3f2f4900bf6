"""Dequantise-then-float64 GEMM and the fused epilogues.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The GEMM and its epilogues have plain definitions, so the oracle is those
definitions written out; the GPU reaches them up to fp32 accumulation order.

* GEMM (fal / Ideogram v4 page, section on epilogue fusion: the GEMM forms
  A @ B tile by tile with on-chip accumulators): C = D(A) @ D(B)^T, with both
  operands dequantised exactly and multiplied in float64.  B is the packed
  weight, stored [N, K] so that its 32-element blocks run along K like A's.
* RMSNorm (same page, epilogue-fusion section and "why head_dim=256 is hard"):
  per row and per head of head_dim contiguous columns,
  y = x * rsqrt(mean(x^2) + eps) * weight.  Reading: eps inside the square
  root, mean over head_dim, weight per column, columns past n_norm_cols pass
  through unchanged (the V part of a fused QKV projection).
* SwiGLU (same page, gated-SiLU section): output = SiLU(C[:, :N/2]) *
  C[:, N/2:], SiLU(z) = z * sigmoid(z); the weight columns are permuted once
  at packing time so that gate and up columns become neighbours.  The oracle
  computes from the logical (un-permuted) halves, so its result does not
  depend on the permutation.
* SwiGLU -> block transform -> MXFP4 (the same page's point that an epilogue
  saves the output's HBM round trip, applied to the FFN's down projection,
  whose input is transformed block by block before quantisation per the
  KroQuant page, "Background and overview" and "Deep analysis"): the SwiGLU
  output h is multiplied, 32 columns at a time, by the down layer's T_b and
  the product is quantised.  Reading: h is carried unrounded between the
  steps (as the re-quantisation takes h itself, not a bf16 copy of it).
"""

import numpy as np

from . import mxfp4, transform


def gemm(a_codes, a_scales, b_codes, b_scales):
    """C[M, N] = D(A) @ D(B)^T in float64.  Codes unpacked [rows, K]."""
    da = mxfp4.dequantize(a_codes, a_scales)
    db = mxfp4.dequantize(b_codes, b_scales)
    return np.matmul(da, db.T)


def epilogue_none(c):
    """No epilogue: the accumulator itself (rounded by the caller's store)."""
    return np.asarray(c, dtype=np.float64)


def rmsnorm_head(c, head_dim, n_norm_cols, weight, eps):
    """Per-head RMSNorm over the first n_norm_cols columns of c.

    c: [M, N] float64; weight: [n_norm_cols] per-column gains.
    """
    c = np.asarray(c, dtype=np.float64)
    m, n = c.shape
    if n_norm_cols % head_dim or n_norm_cols > n:
        raise ValueError("n_norm_cols must be a multiple of head_dim and <= N")
    y = c.copy()
    heads = c[:, :n_norm_cols].reshape(m, n_norm_cols // head_dim, head_dim)
    ms = np.mean(heads * heads, axis=2, keepdims=True)
    rstd = 1.0 / np.sqrt(ms + eps)
    w = np.asarray(weight, dtype=np.float64).reshape(n_norm_cols // head_dim, head_dim)
    y[:, :n_norm_cols] = (heads * rstd * w[None]).reshape(m, n_norm_cols)
    return y


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64 libm exp."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(c_gate, c_up):
    """h = SiLU(gate) * up, elementwise, from the logical halves."""
    return silu(c_gate) * np.asarray(c_up, dtype=np.float64)


def interleave_columns(n_half, group):
    """Physical column order of the gate/up interleave with group size g.

    Returns (pair, is_up) for every physical column p in [0, 2*n_half):
    physical columns come in runs of g gate columns followed by the g up
    columns of the same logical outputs, so pair = (p // 2g) * g + p % g and
    the column is an up column iff (p // g) is odd.  g = 1 gives
    [gate0, up0, gate1, up1, ...].
    """
    if n_half % group:
        raise ValueError("n_half must be a multiple of the group size")
    p = np.arange(2 * n_half)
    pair = (p // (2 * group)) * group + p % group
    is_up = (p // group) % 2 == 1
    return pair, is_up


def interleave_weight(w_gate, w_up, group):
    """Logical [K, N/2] gate and up weights -> physical [K, N] (columns)."""
    w_gate = np.asarray(w_gate)
    w_up = np.asarray(w_up)
    pair, is_up = interleave_columns(w_gate.shape[1], group)
    return np.where(is_up[None, :], w_up[:, pair], w_gate[:, pair])


def swiglu_from_interleaved(c_phys, group):
    """SwiGLU applied to a physical (interleaved) accumulator [M, N]."""
    c_phys = np.asarray(c_phys, dtype=np.float64)
    n_half = c_phys.shape[1] // 2
    pair, is_up = interleave_columns(n_half, group)
    gate = np.empty((c_phys.shape[0], n_half))
    up = np.empty((c_phys.shape[0], n_half))
    gate[:, pair[~is_up]] = c_phys[:, ~is_up]
    up[:, pair[is_up]] = c_phys[:, is_up]
    return swiglu(gate, up)


def requantize(h, return_scaled=False):
    """MXFP4 re-quantisation of an epilogue output along its columns."""
    return mxfp4.quantize(h, return_scaled=return_scaled)


def swiglu_transform_requantize(c_gate, c_up, t, return_scaled=False):
    """h = SwiGLU(gate, up); y = h block-transformed by T (y_b = h_b @ T_b);
    MXFP4 codes and scales of y, all in float64 with h unrounded."""
    return mxfp4.quantize(transform.block_transform(swiglu(c_gate, c_up), t), return_scaled=return_scaled)
