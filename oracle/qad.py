"""Fake quantisation for quantisation-aware distillation (QAD).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: fal / Ideogram v4 page, QAD section.  The student model learns
through its own quantisation: in the forward pass a tensor goes through the
FP4 rounding, so the quantisation noise propagates; in the backward pass the
rounding is cut out of the autodiff graph (its derivative is zero almost
everywhere) and a straight-through estimator passes the gradient on at full
precision.

* Forward: y = D(Q(x)), the value x takes after MXFP4 quantisation (the
  encoding of oracle/mxfp4.py, blocks of 32 along the last axis).
* Backward (reading: the plain straight-through estimator, no clipping to the
  representable range, as the page routes the gradient around the rounding
  unchanged): dL/dx = dL/dy.
"""

import numpy as np

from . import mxfp4


def fake_quantize(x):
    """Forward: MXFP4 quantise then dequantise, float64 result (exact)."""
    codes, scales = mxfp4.quantize(x)
    return mxfp4.dequantize(codes, scales)


def ste_backward(grad_y):
    """Backward: the straight-through estimator passes the gradient as is."""
    return np.array(grad_y, dtype=np.float64, copy=True)
