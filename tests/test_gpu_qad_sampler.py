"""GPU parity of the QAD fake quantisation (bit-exact: its result is unique)
and of the ETD1 / ETD2 / Richardson sampler updates (within the rounding
bound of fp32 arithmetic and one rounding into the storage type)."""

import math

import numpy as np
import pytest
import torch

import golden_io
from gpu_util import announce, dev
from fp4_diffusion_transformer_amd import ops
from oracle import qad, sampler

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------- QAD --
def _bits(t):
    """Bit patterns of a float32 / bfloat16 device tensor (uint32 / uint16)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def _ref_bits(y64, dtype):
    f = y64.astype(np.float32)                        # exact: the values have <= 2 significant bits
    assert np.array_equal(f.astype(np.float64), y64)
    u = f.view(np.uint32)
    if dtype == torch.bfloat16:
        assert not (u & 0xFFFF).any()
        return (u >> 16).astype(np.uint16)
    return u


def _fq_inputs():
    rng = np.random.default_rng(100)
    x = rng.standard_normal((96, 384)) * 2.0 ** rng.integers(-30, 30, (96, 1))
    x[:, rng.choice(384, 6, replace=False)] *= 25
    x[0, :64] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = rng.standard_normal(32) * 2.0 ** -133         # subnormal block: scale byte 0 or 1
    x[3, :32] = rng.standard_normal(32) * 2.0 ** -126
    x[4, :32] = rng.standard_normal(32) * 2.0 ** 120
    return x


@pytest.mark.parametrize("x_dtype,y_dtype", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                             (torch.float32, torch.bfloat16), (torch.bfloat16, torch.float32)])
def test_fake_quant_bit_exact(x_dtype, y_dtype):
    x = _fq_inputs()
    xd = dev(x, x_dtype)
    x_exact = xd.float().cpu().numpy().astype(np.float64)        # the values the kernel reads
    ref = qad.fake_quantize(x_exact)
    announce("fake quant", x_dtype, y_dtype)
    y = ops.fake_quantize_mxfp4(xd, y_dtype=y_dtype)
    assert np.array_equal(_bits(y), _ref_bits(ref, y_dtype))


def test_fake_quant_hand_blocks_every_bf16_value_and_in_place():
    blocks = [b for b in golden_io.mxfp4_blocks() if b[2] != 255]
    hand = np.array([b[1] for b in blocks])
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)].astype(np.float64)
    vals = np.concatenate([vals, np.zeros((-len(vals)) % 256)]).reshape(-1, 256)
    for x in (hand, vals):
        ref = qad.fake_quantize(x)
        announce("fake quant table", x.shape)
        xd = dev(x, torch.bfloat16)
        y = ops.fake_quantize_mxfp4(xd, out=xd)                   # in place
        assert np.array_equal(_bits(xd), _ref_bits(ref, torch.bfloat16))


def test_fake_quant_ragged_rows_empty_and_nonfinite():
    rng = np.random.default_rng(101)
    x = rng.standard_normal((333, 96))
    ref = qad.fake_quantize(x)
    announce("fake quant ragged")
    y = ops.fake_quantize_mxfp4(dev(x, torch.float32))
    assert np.array_equal(_bits(y), _ref_bits(ref, torch.float32))
    e = ops.fake_quantize_mxfp4(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.shape == (0, 64)
    # a block holding Inf or NaN comes back as NaN (documented; not part of the oracle)
    x[5, 40] = np.inf
    x[6, 3] = np.nan
    y = ops.fake_quantize_mxfp4(dev(x, torch.float32)).cpu().numpy()
    assert np.isnan(y[5, 32:64]).all() and np.isnan(y[6, :32]).all()
    assert np.isfinite(y[5, :32]).all() and np.isfinite(y[5, 64:]).all()


def test_fake_quant_straight_through_gradient():
    rng = np.random.default_rng(102)
    x = dev(rng.standard_normal((64, 128)) * 3, torch.float32).requires_grad_(True)
    g = dev(rng.standard_normal((64, 128)), torch.float32)
    announce("fake quant STE")
    y = ops.fake_quantize_ste(x)
    assert np.array_equal(_bits(y.detach()), _ref_bits(qad.fake_quantize(x.detach().cpu().numpy().astype(
        np.float64)), torch.float32))
    (y * g).sum().backward()
    assert torch.equal(x.grad, g)                                  # dL/dx = dL/dy exactly


# --------------------------------------------------------------- sampler --
# half an ulp, relative: 24, 8 and 11 significant bits
_REL = {torch.float32: 2.0 ** -24, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
_ABS = {torch.float32: 2.0 ** -150, torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}


def _vp(t):
    a = math.cos(0.5 * math.pi * t)
    return a, math.sqrt(1.0 - a * a)


def _stored(rng, n, dtype, scale=1.0):
    t = dev(rng.standard_normal(n) * scale, dtype)
    return t, t.float().cpu().numpy().astype(np.float64)


def _check(out, ref, mag, dtype, what):
    """|out - ref| <= e32 + half an output ulp, e32 = 3 * 2^-24 * mag (two fp32
    roundings of terms summing to mag in magnitude)."""
    g = out.float().cpu().numpy().astype(np.float64)
    e32 = 3 * 2.0 ** -24 * mag
    bound = e32 + _REL[dtype] * (np.abs(ref) + e32) + _ABS[dtype]
    bad = np.abs(g - ref) > bound
    assert not bad.any(), "%s: %d of %d outside the bound, first %d: gpu %r ref %r" % (
        what, int(bad.sum()), bad.size, int(np.argmax(bad)), g[np.argmax(bad)], ref[np.argmax(bad)])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("n", [1, 7, 8, 4099, 1 << 18])
def test_etd_updates(dtype, n):
    rng = np.random.default_rng(n + 7)
    (x, xh), (x0, x0h), (xp, xph) = (_stored(rng, n, dtype) for _ in range(3))
    d1, c, _ = ops.etd_coefficients(*_vp(0.6), *_vp(0.5), order=1)
    d, c0, c1 = ops.etd_coefficients(*_vp(0.6), *_vp(0.5), order=2, first_step=False)
    k = [float(np.float32(v)) for v in (d1, c, d, c0, c1)]        # the fp32 scalars the kernel gets
    announce("etd1/etd2", dtype, n)
    out1 = ops.etd1_update(x, x0, d1, c)
    out2 = ops.etd2_update(x, x0, xp, d, c0, c1)
    _check(out1, sampler.etd1_update(xh, x0h, k[0], k[1]), np.abs(k[0] * xh) + np.abs(k[1] * x0h), dtype, "etd1")
    _check(out2, sampler.etd2_update(xh, x0h, xph, k[2], k[3], k[4]),
           np.abs(k[2] * xh) + np.abs(k[3] * x0h) + np.abs(k[4] * xph), dtype, "etd2")
    # in place on x, as a sampler loop runs it
    ops.etd1_update(x, x0, d1, c, out=x)
    _check(x, sampler.etd1_update(xh, x0h, k[0], k[1]), np.abs(k[0] * xh) + np.abs(k[1] * x0h), dtype, "etd1 inplace")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("p", [1, 2])
def test_richardson_combine(dtype, p):
    rng = np.random.default_rng(20 + p)
    n = 100003
    fine, fh = _stored(rng, n, dtype)
    coarse, ch = _stored(rng, n, dtype)
    scale = 2.0 ** p
    announce("richardson", dtype, p)
    out = ops.richardson_combine(fine, coarse, scale)
    mag = (np.abs(scale * fh) + np.abs(ch)) / (scale - 1) + np.abs(sampler.richardson_combine(fh, ch, scale))
    _check(out, sampler.richardson_combine(fh, ch, scale), mag, dtype, "richardson")


def test_etd1_sampler_loop_is_exact_for_a_constant_prediction():
    """Twelve chained ETD1 steps in fp32 on the device against the closed
    form of the exact solution (constant data prediction)."""
    rng = np.random.default_rng(30)
    n = 1 << 16
    x, xh = _stored(rng, n, torch.float32)
    x0, x0h = _stored(rng, n, torch.float32)
    ts = np.linspace(0.95, 0.02, 13)
    announce("etd1 loop")
    for s, t in zip(ts[:-1], ts[1:]):
        d, c, _ = ops.etd_coefficients(*_vp(s), *_vp(t))
        ops.etd1_update(x, x0, d, c, out=x)
    a0, s0 = _vp(ts[0])
    a1, s1 = _vp(ts[-1])
    exact = (s1 / s0) * xh + s1 * (a1 / s1 - a0 / s0) * x0h
    g = x.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - exact)) <= 1e-5 * (np.max(np.abs(xh)) + np.max(np.abs(x0h)))


# ----------------------------------------------------- at the bench's sizes --
def test_fake_quant_bench_shape_bit_exact():
    """The QAD forward at the size bench.py times (4096 x 3072 bf16 -> bf16),
    every element against the oracle."""
    rng = np.random.default_rng(101)
    x = rng.standard_normal((4096, 3072)) * 2.0 ** rng.integers(-8, 9, (4096, 1))
    xd = dev(x, torch.bfloat16)
    x_exact = xd.float().cpu().numpy().astype(np.float64)
    announce("fake quant bench shape", x.shape)
    y = ops.fake_quantize_mxfp4(xd, y_dtype=torch.bfloat16)
    assert np.array_equal(_bits(y), _ref_bits(qad.fake_quantize(x_exact), torch.bfloat16))


def test_sampler_updates_bench_shape():
    """ETD1, ETD2 and the Richardson combine on the latent bench.py times
    (16 latents of 16 x 128 x 128 fp32), every element within the bound."""
    n = 16 * 16 * 128 * 128
    rng = np.random.default_rng(102)
    (x, xh), (x0, x0h), (xp, xph) = (_stored(rng, n, torch.float32) for _ in range(3))
    d1, c, _ = ops.etd_coefficients(*_vp(0.6), *_vp(0.5), order=1)
    d, c0, c1 = ops.etd_coefficients(*_vp(0.6), *_vp(0.5), order=2, first_step=False)
    k = [float(np.float32(v)) for v in (d1, c, d, c0, c1)]
    announce("sampler bench shape", n)
    _check(ops.etd1_update(x, x0, d1, c), sampler.etd1_update(xh, x0h, k[0], k[1]),
           np.abs(k[0] * xh) + np.abs(k[1] * x0h), torch.float32, "etd1 bench shape")
    _check(ops.etd2_update(x, x0, xp, d, c0, c1), sampler.etd2_update(xh, x0h, xph, k[2], k[3], k[4]),
           np.abs(k[2] * xh) + np.abs(k[3] * x0h) + np.abs(k[4] * xph), torch.float32, "etd2 bench shape")
    out = ops.richardson_combine(x, x0, 2.0)
    mag = (np.abs(2.0 * xh) + np.abs(x0h)) + np.abs(sampler.richardson_combine(xh, x0h, 2.0))
    _check(out, sampler.richardson_combine(xh, x0h, 2.0), mag, torch.float32, "richardson bench shape")
