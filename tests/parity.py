"""Comparison rules between the HIP path and the CPU oracle.

Values: err_i = |g_i - r_i| / max(|r_i|, 0.1 * RMS(r over the row, or over
the row's head)), so cancellation near zero does not blow up the relative
error.  Bars: 2e-3 for fp32 stores, 1e-2 after a bf16 store (fp32
accumulation of K products of magnitude ~1 differs from float64 by about
sqrt(K) * 2**-24 of the row RMS, some 100x below the bars; bf16 rounding
alone is 2**-9 relative).

Codes: plain quantisation of given inputs has exactly one correct result and
is compared bit for bit.  Where the value being quantised is itself an fp32
sum (transform output, SwiGLU output), a code may differ from the float64
oracle only where the oracle's scaled value lies within TAU of a rounding
midpoint, and a block scale only where the block amax lies within relative
AMAX_REL of a power of two (then the whole block is excused).  fp32 sums are
off by ~1e-5 in scaled units, so TAU leaves a ~10x margin; everything else
must match exactly.
"""

import numpy as np

from oracle import gemm as ogemm
from oracle import mxfp4
from oracle import transform as otransform

TAU = 1e-4
AMAX_REL = 1e-5
TOL_F32 = 2e-3
TOL_BF16 = 1e-2


def rel_err(gpu, ref, group=None):
    """Max S14-style relative error; group = columns per RMS group (None: whole row)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    m, n = r.shape
    grp = n if group is None else group
    rr = r.reshape(m, n // grp, grp)
    rms = np.sqrt(np.mean(rr * rr, axis=2, keepdims=True))
    floor = np.broadcast_to(0.1 * rms, rr.shape).reshape(m, n)
    denom = np.maximum(np.abs(r), floor)
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(g - r) / denom))


def assert_close(gpu, ref, tol, group=None, what="", mask=None):
    """rel_err over all elements, or over those where `mask` is set (the
    RMS floor still comes from the whole row or head of the reference)."""
    if mask is None:
        e = rel_err(gpu, ref, group)
    else:
        g = np.asarray(gpu, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        m, n = r.shape
        grp = n if group is None else group
        rr = r.reshape(m, n // grp, grp)
        rms = np.sqrt(np.mean(rr * rr, axis=2, keepdims=True))
        denom = np.maximum(np.abs(r), np.broadcast_to(0.1 * rms, rr.shape).reshape(m, n))
        denom = np.where(denom == 0, 1.0, denom)
        err = np.abs(g - r) / denom
        e = float(np.max(err[mask])) if np.any(mask) else 0.0
    assert e <= tol, "%s: max relative error %.3e > %.1e" % (what, e, tol)
    return e


def unpack(packed):
    return mxfp4.unpack_codes(np.asarray(packed, dtype=np.uint8))


def assert_codes_exact(gpu_packed, gpu_scales, ref_codes, ref_scales, what=""):
    gc = unpack(gpu_packed)
    gs = np.asarray(gpu_scales, dtype=np.uint8)
    bad_s = np.argwhere(gs != ref_scales)
    assert bad_s.size == 0, "%s: %d scale mismatches, first at %s: gpu %d ref %d" % (
        what, len(bad_s), bad_s[0], gs[tuple(bad_s[0])], ref_scales[tuple(bad_s[0])])
    bad = np.argwhere(gc != ref_codes)
    assert bad.size == 0, "%s: %d code mismatches, first at %s: gpu %d ref %d" % (
        what, len(bad), bad[0], gc[tuple(bad[0])], ref_codes[tuple(bad[0])])


def _near_midpoint(q, tau=TAU):
    a = np.abs(q)
    near = np.zeros(a.shape, dtype=bool)
    for mid in mxfp4.E2M1_MIDPOINTS:
        near |= np.abs(a - mid) <= tau
    return near


def _near_pow2(amax, amax_rel=AMAX_REL):
    with np.errstate(divide="ignore"):
        e = np.round(np.log2(np.where(amax > 0, amax, 1.0)))
    return np.abs(amax / 2.0 ** e - 1.0) <= amax_rel


def assert_codes_banded(gpu_packed, gpu_scales, ref_values, what="", ref=None, tau=TAU, amax_rel=AMAX_REL):
    """Codes of fp32 sums vs the float64 oracle values, with the excusal band.

    ref: optionally the oracle's mxfp4.quantize(ref_values, return_scaled=True)
    if already computed; tau: the midpoint band, a scalar or one per element;
    amax_rel: the power-of-two band of block amaxes, a scalar or one per block.
    Returns (excused_codes, excused_blocks) counts."""
    ref_values = np.asarray(ref_values, dtype=np.float64)
    rc, rs, q = ref if ref is not None else mxfp4.quantize(ref_values, return_scaled=True)
    gc = unpack(gpu_packed)
    gs = np.asarray(gpu_scales, dtype=np.uint8)
    m, n = ref_values.shape
    amax = np.max(np.abs(ref_values.reshape(m, n // 32, 32)), axis=2)
    scale_bad = gs != rs
    scale_ok_excuse = _near_pow2(amax, amax_rel)
    unexcused_scale = scale_bad & ~scale_ok_excuse
    assert not unexcused_scale.any(), "%s: %d unexcused scale mismatches at %s" % (
        what, int(unexcused_scale.sum()), np.argwhere(unexcused_scale)[0])
    block_excused = np.repeat(scale_bad, 32, axis=1)
    code_bad = (gc != rc) & ~block_excused
    unexcused = code_bad & ~_near_midpoint(q, tau)
    assert not unexcused.any(), "%s: %d unexcused code mismatches, first %s (ref q=%r)" % (
        what, int(unexcused.sum()), np.argwhere(unexcused)[0], q[tuple(np.argwhere(unexcused)[0])])
    return int(code_bad.sum()), int(scale_bad.sum())


def assert_fused_codes(gpu_codes, gpu_scales, c_gate, c_up, t, what=""):
    """Unpacked-row codes / scales of the fused SwiGLU -> block transform ->
    MXFP4 epilogue against the oracle's, from the oracle's accumulators
    c_gate, c_up (float64) and T, with the plain midpoint band (the kernel
    carries the fp32 h exactly, as three bf16 parts, so only the order of
    its fp32 sums differs).  Returns (h, y_ref, excused codes, excused
    blocks)."""
    t64 = np.asarray(t, dtype=np.float64)
    rc, rs, q = ogemm.swiglu_transform_requantize(c_gate, c_up, t64, return_scaled=True)
    h = ogemm.swiglu(c_gate, c_up)
    y_ref = otransform.block_transform(h, t64)
    exc, blk = assert_codes_banded(gpu_codes, gpu_scales, y_ref, what, ref=(rc, rs, q))
    assert exc <= 0.001 * y_ref.size and blk <= 0.001 * rs.size, "%s: %d codes / %d blocks excused" % (what, exc, blk)
    return h, y_ref, exc, blk
