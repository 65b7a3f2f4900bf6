"""GPU parity of the fused MXFP4 GEMM + epilogues against the oracle.

Operands are MXFP4 codes produced by the oracle's quantiser from seeded
inputs, so these tests isolate the GEMM and its epilogues.  Shapes span
several workgroup tiles and a ragged last token tile.
"""

import numpy as np
import pytest
import torch

import layout
import parity
from gpu_util import announce, dev, dev_u8, host
from fp4_diffusion_transformer_amd import ops, workloads
from oracle import bf16 as obf16
from oracle import gemm as ogemm
from oracle import mxfp4
from oracle import transform as otransform

pytestmark = pytest.mark.gpu


def _operands(rng, m, n, k, spread=True):
    x = rng.standard_normal((m, k))
    if spread:
        x *= 2.0 ** rng.integers(-3, 4, (m, 1))
    w = rng.standard_normal((n, k)) / np.sqrt(k)
    ac, as_ = mxfp4.quantize(x)
    bc, bs = mxfp4.quantize(w)
    return ac, as_, bc, bs


def _mx(codes, scales):
    """Oracle codes (unpacked, row-major) -> tiled MxTensor on the device."""
    rows, cols = codes.shape
    return ops.MxTensor(dev_u8(layout.tile_codes(mxfp4.pack_codes(codes))), dev_u8(layout.tile_scales(scales)),
                        rows, cols, "tiled")


def _dev_ops(ac, as_, bc, bs):
    return _mx(ac, as_), _mx(bc, bs)


def test_exact_on_representable_inputs():
    """Grid values with equal scales: every partial sum is exact in fp32, so
    the fp32 output must equal the oracle bit for bit."""
    rng = np.random.default_rng(0)
    m, n, k = 300, 512, 4096
    ac = rng.integers(0, 16, (m, k)).astype(np.uint8)
    bc = rng.integers(0, 16, (n, k)).astype(np.uint8)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    ref = ogemm.gemm(ac, as_, bc, bs)
    announce("gemm none exact", m, n, k)
    out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=torch.float32)
    assert np.array_equal(host(out).astype(np.float64), ref)


def test_scales_apply_per_block_and_operand():
    """Distinct scale per (row, K-block) on each side, exact products: any
    mix-up of the scale bytes between K-steps, lane groups or operands shows."""
    rng = np.random.default_rng(1)
    m, n, k = 64, 256, 1024
    ac = rng.integers(0, 16, (m, k)).astype(np.uint8)
    bc = rng.integers(0, 16, (n, k)).astype(np.uint8)
    as_ = rng.integers(124, 131, (m, k // 32)).astype(np.uint8)
    bs = rng.integers(124, 131, (n, k // 32)).astype(np.uint8)
    ref = ogemm.gemm(ac, as_, bc, bs)
    announce("gemm none scales", m, n, k)
    out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=torch.float32)
    parity.assert_close(host(out), ref, 1e-5, what="per-block scales")


@pytest.mark.parametrize("m", [1, 255, 256, 257, 600])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_none_random(m, out_dtype):
    rng = np.random.default_rng(m)
    n, k = 768, 768
    ac, as_, bc, bs = _operands(rng, m, n, k)
    ref = ogemm.gemm(ac, as_, bc, bs)
    announce("gemm none", m, n, k, out_dtype)
    out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=out_dtype)
    tol = parity.TOL_F32 if out_dtype == torch.float32 else parity.TOL_BF16
    parity.assert_close(host(out), ref, tol, what="none")
    if out_dtype == torch.bfloat16:
        # within one bf16 rounding of the RNE-rounded reference
        assert np.max(np.abs(host(out) - obf16.round_bf16(ref)) / np.maximum(np.abs(ref), 1e-3)) < 2 ** -7


@pytest.mark.parametrize("head_dim,n,n_norm", [(128, 768, 512), (128, 768, 384), (128, 512, 0),
                                              (256, 768, 512), (256, 512, 256)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_rmsnorm_head(head_dim, n, n_norm, out_dtype):
    rng = np.random.default_rng(head_dim + n + n_norm)
    m, k = 300, 512
    ac, as_, bc, bs = _operands(rng, m, n, k)
    norm_w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
    eps = 1e-6
    c = ogemm.gemm(ac, as_, bc, bs)
    ref = ogemm.rmsnorm_head(c, head_dim, n_norm, norm_w.astype(np.float64), eps)
    announce("gemm rmsnorm", head_dim, n, n_norm, out_dtype)
    out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), head_dim, n_norm,
                                             dev(norm_w, torch.float32) if n_norm else None, eps,
                                             out_dtype=out_dtype)
    tol = parity.TOL_F32 if out_dtype == torch.float32 else parity.TOL_BF16
    parity.assert_close(host(out), ref, tol, group=head_dim, what="rmsnorm hd%d" % head_dim)


def test_rmsnorm_eps_dominates_tiny_heads():
    """Heads whose accumulators are tiny: the eps term decides the scale."""
    rng = np.random.default_rng(3)
    m, n, k = 64, 256, 256
    ac, as_, bc, bs = _operands(rng, m, n, k, spread=False)
    as_ = np.full_like(as_, 127 - 12)            # accumulators ~2**-12
    norm_w = np.ones(n, np.float32)
    eps = 1e-6
    ref = ogemm.rmsnorm_head(ogemm.gemm(ac, as_, bc, bs), 128, n, norm_w.astype(np.float64), eps)
    announce("gemm rmsnorm tiny heads")
    out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), 128, n, dev(norm_w, torch.float32),
                                             eps, out_dtype=torch.float32)
    parity.assert_close(host(out), ref, parity.TOL_F32, group=128, what="tiny heads")


def _swiglu_operands(rng, m, n_half, k, parts=False):
    x = rng.standard_normal((m, k)) * 2.0 ** rng.integers(-2, 3, (m, 1))
    wg = rng.standard_normal((k, n_half)) / np.sqrt(k) * 2
    wu = rng.standard_normal((k, n_half)) / np.sqrt(k)
    ac, as_ = mxfp4.quantize(x)
    gc_, gs_ = mxfp4.quantize(wg.T)
    uc_, us_ = mxfp4.quantize(wu.T)
    g = ops.swiglu_interleave_group()
    # physical weight rows: the oracle's codes of the logical columns, interleaved
    pair, is_up = ogemm.interleave_columns(n_half, g)
    bc = np.where(is_up[:, None], uc_[pair], gc_[pair])
    bs = np.where(is_up[:, None], us_[pair], gs_[pair])
    c_g = ogemm.gemm(ac, as_, gc_, gs_)
    c_u = ogemm.gemm(ac, as_, uc_, us_)
    if parts:
        return (ac, as_, bc, bs), c_g, c_u
    return (ac, as_, bc, bs), ogemm.swiglu(c_g, c_u)


@pytest.mark.parametrize("m", [300, 1])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_swiglu_values(m, out_dtype):
    rng = np.random.default_rng(11 + m)
    operands, h_ref = _swiglu_operands(rng, m, 384, 512)
    announce("gemm swiglu", m, out_dtype)
    h, mx = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=out_dtype, requant=False)
    assert mx is None
    tol = parity.TOL_F32 if out_dtype == torch.float32 else parity.TOL_BF16
    parity.assert_close(host(h), h_ref, tol, what="swiglu")


@pytest.mark.parametrize("with_bf16", [False, True])
def test_swiglu_requant(with_bf16):
    rng = np.random.default_rng(21)
    operands, h_ref = _swiglu_operands(rng, 300, 512, 768)
    announce("gemm swiglu requant", with_bf16)
    h, mx = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=torch.bfloat16 if with_bf16 else None,
                                         requant=True)
    if with_bf16:
        parity.assert_close(host(h), h_ref, parity.TOL_BF16, what="swiglu bf16 + requant")
    else:
        assert h is None
    codes = layout.untile_codes(host(mx.codes), mx.rows, mx.cols)
    scales = layout.untile_scales(host(mx.scales), mx.rows, mx.cols)
    exc_codes, exc_blocks = parity.assert_codes_banded(codes, scales, h_ref, "swiglu requant")
    assert exc_codes <= 0.001 * h_ref.size


@pytest.mark.parametrize("k", [512, 256])
@pytest.mark.parametrize("epilogue", ["none", "rmsnorm", "rmsnorm256", "swiglu_requant"])
def test_persistent_many_tiles_ragged(epilogue, k):
    """More 256 x 256 tiles (4 x 80 = 320) than a persistent grid holds, so
    workgroups run several tiles in turn (the next tile's loads overlapping
    the epilogue), with a ragged last token tile (1000 = 3 * 256 + 232).  On
    a 256-CU device the plain and RMSNorm epilogues run the partial second
    round (64 tiles) as 256 quarter tiles of 64 tokens.  K = 256 is the
    shortest K: two stages, fewer than the quarter tiles keep in flight."""
    rng = np.random.default_rng(31)
    m, n = 1000, 256 * 80
    rows = np.unique(np.concatenate([[0, 255, 256, 767, 768, 999], rng.choice(m, 40, replace=False)]))
    announce("gemm persistent", epilogue, m, n, k)
    if epilogue == "swiglu_requant":
        operands, h_ref = _swiglu_operands(rng, m, n // 2, k)
        _, mx = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=None, requant=True)
        codes = layout.untile_codes(host(mx.codes), mx.rows, mx.cols)
        scales = layout.untile_scales(host(mx.scales), mx.rows, mx.cols)
        exc, _ = parity.assert_codes_banded(codes[rows], scales[rows], h_ref[rows], "persistent swiglu requant")
        assert exc <= 0.001 * h_ref[rows].size
        return
    ac, as_, bc, bs = _operands(rng, m, n, k)
    c = ogemm.gemm(ac[rows], as_[rows], bc, bs)
    if epilogue == "none":
        out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=torch.float32)
        parity.assert_close(host(out)[rows], c, parity.TOL_F32, what="persistent none")
    else:
        hd = 256 if epilogue == "rmsnorm256" else 128
        n_norm = n - 2048
        norm_w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
        ref = ogemm.rmsnorm_head(c, hd, n_norm, norm_w.astype(np.float64), 1e-6)
        out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), hd, n_norm,
                                                 dev(norm_w, torch.float32), 1e-6, out_dtype=torch.bfloat16)
        parity.assert_close(host(out)[rows], ref, parity.TOL_BF16, group=hd, what="persistent " + epilogue)


@pytest.mark.parametrize("epilogue", ["none", "rmsnorm"])
def test_quarter_tiles_two_per_workgroup(epilogue):
    """384 tiles (4 x 96) on a 256-CU grid leave a partial round of 128
    tiles: 512 quarter tiles, two per workgroup in turn (the second one's
    loads start after the first one's epilogue has used the ring), K = 768
    (six stages: one full turn of the quarter loop's unrolled body), and a
    ragged last token tile."""
    rng = np.random.default_rng(37)
    m, n, k = 1000, 256 * 96, 768
    rows = np.unique(np.concatenate([[0, 63, 64, 255, 768, 831, 832, 999], rng.choice(m, 40, replace=False)]))
    announce("gemm quarter x2", epilogue, m, n, k)
    ac, as_, bc, bs = _operands(rng, m, n, k)
    c = ogemm.gemm(ac[rows], as_[rows], bc, bs)
    if epilogue == "none":
        out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=torch.bfloat16)
        parity.assert_close(host(out)[rows], c, parity.TOL_BF16, what="quarter x2 none")
    else:
        n_norm = n - 1024
        norm_w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
        ref = ogemm.rmsnorm_head(c, 128, n_norm, norm_w.astype(np.float64), 1e-6)
        out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), 128, n_norm,
                                                 dev(norm_w, torch.float32), 1e-6, out_dtype=torch.bfloat16)
        parity.assert_close(host(out)[rows], ref, parity.TOL_BF16, group=128, what="quarter x2 rmsnorm")


# SwiGLU -> down-projection block transform -> MXFP4, fused in the epilogue

def _check_fused(mx, y, c_g, c_u, t, rows=None, what="fused"):
    """Codes (and y, if stored) of the fused epilogue against the oracle's
    SwiGLU -> transform -> quantise, on the given rows."""
    if rows is None:
        rows = np.arange(c_g.shape[0])
    codes = layout.untile_codes(host(mx.codes), mx.rows, mx.cols)[rows]
    scales = layout.untile_scales(host(mx.scales), mx.rows, mx.cols)[rows]
    h_rows, y_ref, _, _ = parity.assert_fused_codes(codes, scales, c_g[rows], c_u[rows], t, what)
    if y is not None:
        yg = host(y)[rows].astype(np.float64)
        parity.assert_close(yg, y_ref, parity.TOL_F32, what=what + " y")
        # y from the fp32 h carried exactly: besides h's own fp32 error (from
        # the GEMM's sums and the SiLU, a few 2^-24 relative), only the fp32
        # summation order; a bf16-rounded h (error up to 2^-9 |h|) or a
        # two-part split (up to 2^-16 |h|) can exceed this
        mag = otransform.block_transform(np.abs(h_rows), np.abs(t.astype(np.float64)))
        rms = np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True))
        assert np.all(np.abs(yg - y_ref) <= 2.0 ** -18 * mag + 1e-5 * rms), what + ": y outside the bound"


@pytest.mark.parametrize("m,n_t", [(300, 8), (300, 1), (1, 8)])
def test_swiglu_transform(m, n_t):
    rng = np.random.default_rng(51 + m + n_t)
    operands, c_g, c_u = _swiglu_operands(rng, m, 256, 512, parts=True)
    t = workloads.transforms(60 + n_t, n_t)
    announce("gemm swiglu transform", m, n_t)
    y, mx = ops.gemm_fp4_epilogue_swiglu_transform(*_dev_ops(*operands), dev(t, torch.bfloat16),
                                                   y_dtype=torch.float32)
    _check_fused(mx, y, c_g, c_u, t, what="swiglu transform")


def test_swiglu_transform_codes_only_and_bf16_y():
    """Codes without y, and with a bf16 y: the codes do not depend on it."""
    rng = np.random.default_rng(57)
    operands, c_g, c_u = _swiglu_operands(rng, 300, 512, 768, parts=True)
    t = workloads.transforms(61, 16)
    announce("gemm swiglu transform codes only / bf16 y")
    a, b = _dev_ops(*operands)
    y0, mx0 = ops.gemm_fp4_epilogue_swiglu_transform(a, b, dev(t, torch.bfloat16))
    assert y0 is None
    _check_fused(mx0, None, c_g, c_u, t, what="swiglu transform codes")
    y1, mx1 = ops.gemm_fp4_epilogue_swiglu_transform(a, b, dev(t, torch.bfloat16), y_dtype=torch.bfloat16)
    # (the padding rows of the tiled buffers are never written: compare the rows)
    assert np.array_equal(layout.untile_codes(host(mx0.codes), 300, 512),
                          layout.untile_codes(host(mx1.codes), 300, 512))
    assert np.array_equal(layout.untile_scales(host(mx0.scales), 300, 512),
                          layout.untile_scales(host(mx1.scales), 300, 512))
    h_ref = ogemm.swiglu(c_g, c_u)
    parity.assert_close(host(y1), otransform.block_transform(h_ref, t.astype(np.float64)), parity.TOL_BF16,
                        what="swiglu transform bf16 y")


def test_swiglu_transform_identity_is_requant():
    """T = I: the fused codes follow the plain SwiGLU requant of h."""
    rng = np.random.default_rng(58)
    operands, c_g, c_u = _swiglu_operands(rng, 300, 256, 512, parts=True)
    t = np.eye(32, dtype=np.float32)[None]
    announce("gemm swiglu transform identity")
    _, mx = ops.gemm_fp4_epilogue_swiglu_transform(*_dev_ops(*operands), dev(t, torch.bfloat16))
    _check_fused(mx, None, c_g, c_u, t, what="swiglu transform identity")


def test_swiglu_transform_persistent_many_tiles_ragged():
    """320 tiles on the persistent grid, ragged last token tile, one T per
    block (n_t = 320)."""
    rng = np.random.default_rng(59)
    m, n, k = 1000, 256 * 80, 512
    rows = np.unique(np.concatenate([[0, 255, 256, 767, 768, 999], rng.choice(m, 40, replace=False)]))
    operands, c_g, c_u = _swiglu_operands(rng, m, n // 2, k, parts=True)
    t = workloads.transforms(62, n // 64)
    announce("gemm swiglu transform persistent", m, n, k)
    y, mx = ops.gemm_fp4_epilogue_swiglu_transform(*_dev_ops(*operands), dev(t, torch.bfloat16),
                                                   y_dtype=torch.float32)
    _check_fused(mx, y, c_g, c_u, t, rows=rows, what="persistent swiglu transform")


# K a multiple of the 128-deep stage but not of 256: an odd number of K
# stages (the ring's peel then covers 1, 3 or 2 stages)

@pytest.mark.parametrize("k", [384, 640, 1152])
@pytest.mark.parametrize("epilogue", ["none", "rmsnorm256", "swiglu_requant"])
def test_k_odd_stage_count(epilogue, k):
    rng = np.random.default_rng(71 + k)
    m, n = 300, 768
    announce("gemm odd K stages", epilogue, m, n, k)
    if epilogue == "swiglu_requant":
        operands, h_ref = _swiglu_operands(rng, m, n // 2, k)
        h, mx = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=torch.float32, requant=True)
        parity.assert_close(host(h), h_ref, parity.TOL_F32, what="odd K swiglu")
        codes = layout.untile_codes(host(mx.codes), mx.rows, mx.cols)
        scales = layout.untile_scales(host(mx.scales), mx.rows, mx.cols)
        exc, _ = parity.assert_codes_banded(codes, scales, h_ref, "odd K swiglu requant")
        assert exc <= 0.001 * h_ref.size
        return
    ac, as_, bc, bs = _operands(rng, m, n, k)
    c = ogemm.gemm(ac, as_, bc, bs)
    if epilogue == "none":
        out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=torch.float32)
        parity.assert_close(host(out), c, parity.TOL_F32, what="odd K none")
    else:
        norm_w = rng.uniform(0.5, 1.5, 512).astype(np.float32)
        ref = ogemm.rmsnorm_head(c, 256, 512, norm_w.astype(np.float64), 1e-6)
        out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), 256, 512, dev(norm_w, torch.float32),
                                                 1e-6, out_dtype=torch.float32)
        parity.assert_close(host(out), ref, parity.TOL_F32, group=256, what="odd K rmsnorm")


def test_k_odd_stage_count_persistent_quarters():
    """K = 384 on a persistent grid whose partial last round runs as quarter
    tiles (384 tiles = 4 x 96 on 256 CUs), ragged last token tile."""
    rng = np.random.default_rng(79)
    m, n, k = 1000, 256 * 96, 384
    rows = np.unique(np.concatenate([[0, 63, 64, 255, 768, 831, 832, 999], rng.choice(m, 40, replace=False)]))
    announce("gemm odd K persistent quarters", m, n, k)
    ac, as_, bc, bs = _operands(rng, m, n, k)
    c = ogemm.gemm(ac[rows], as_[rows], bc, bs)
    n_norm = n - 1024
    norm_w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
    ref = ogemm.rmsnorm_head(c, 128, n_norm, norm_w.astype(np.float64), 1e-6)
    out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), 128, n_norm, dev(norm_w, torch.float32),
                                             1e-6, out_dtype=torch.bfloat16)
    parity.assert_close(host(out)[rows], ref, parity.TOL_BF16, group=128, what="odd K quarters")


def test_largest_operand_size():
    """The largest M the 32-bit operand offsets allow at K = 256 (the token
    codes just under 2^31 bytes), plain epilogue, bf16 out (an 8.6 GB
    output).  A is a 4096-row block repeated (its tiled bytes repeat every
    2048 row pairs and 128 scale blocks), so the oracle's rows are rows of
    the block; sampled rows at both ends and around 2^24."""
    k, n, blk = 256, 256, 4096
    m = ((2 ** 31 - 1) // (k // 2)) & ~1                  # even: codes of m rows < 2^31 bytes
    m -= m % blk                                           # whole repeats of the block
    assert (m + 1) * (k // 2) <= 2 ** 31 - 1
    rng = np.random.default_rng(83)
    ac, as_, bc, bs = _operands(rng, blk, n, k)
    tc = torch.from_numpy(layout.tile_codes(mxfp4.pack_codes(ac)))
    ts = torch.from_numpy(layout.tile_scales(as_))
    reps = m // blk
    announce("gemm largest operand", m, n, k)
    a = ops.MxTensor(tc.to("cuda").repeat(reps, 1), ts.to("cuda").repeat(reps, 1), m, k, "tiled")
    b = _mx(bc, bs)
    out = ops.gemm_fp4_epilogue_none(a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, blk - 1, blk, m // 2, 2 ** 24 - 1, 2 ** 24, m - blk, m - 2, m - 1],
                                     rng.choice(m, 16, replace=False)]))
    rows = rows[rows < m]
    got = out[torch.from_numpy(rows).to("cuda")].float().cpu().numpy().astype(np.float64)
    del out, a
    ref = ogemm.gemm(ac[rows % blk], as_[rows % blk], bc, bs)
    parity.assert_close(got, ref, parity.TOL_BF16, what="largest operand")
