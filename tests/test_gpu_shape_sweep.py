"""A seeded sweep of GEMM shapes against the oracle, every epilogue.

Shapes are drawn once from a fixed seed: M anywhere in [1, 700] (ragged
token tiles, single rows), N a multiple of the 256-channel tile, K any
multiple of the 128-deep stage from 256 (odd and even stage counts, every
ring peel).  Each case runs the plain (bf16 and fp32), per-head RMSNorm
(hd 128 and 256, random n_norm) and SwiGLU + requant epilogues on oracle
operands, with the same comparison rules as the other GEMM tests.
"""

import numpy as np
import pytest
import torch

import layout
import parity
from gpu_util import announce, dev, host
from fp4_diffusion_transformer_amd import ops
from oracle import gemm as ogemm
from test_gpu_gemm import _dev_ops, _operands, _swiglu_operands

pytestmark = pytest.mark.gpu


def _shapes(n_cases=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        m = int(rng.integers(1, 701))
        n = 256 * int(rng.integers(1, 5))
        k = 128 * int(rng.integers(2, 13))
        out.append((m, n, k))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("m,n,k", SHAPES, ids=["m%d-n%d-k%d" % s for s in SHAPES])
def test_sweep_none(m, n, k):
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    ac, as_, bc, bs = _operands(rng, m, n, k)
    ref = ogemm.gemm(ac, as_, bc, bs)
    for out_dtype, tol in ((torch.float32, parity.TOL_F32), (torch.bfloat16, parity.TOL_BF16)):
        announce("sweep none", m, n, k, out_dtype)
        out = ops.gemm_fp4_epilogue_none(*_dev_ops(ac, as_, bc, bs), out_dtype=out_dtype)
        parity.assert_close(host(out), ref, tol, what="none %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", SHAPES, ids=["m%d-n%d-k%d" % s for s in SHAPES])
def test_sweep_rmsnorm(m, n, k):
    rng = np.random.default_rng(m * 104729 + n * 17 + k)
    ac, as_, bc, bs = _operands(rng, m, n, k)
    c = ogemm.gemm(ac, as_, bc, bs)
    eps = 1e-6
    for head_dim in (128, 256):
        n_norm = head_dim * int(rng.integers(0, n // head_dim + 1))
        norm_w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
        ref = ogemm.rmsnorm_head(c, head_dim, n_norm, norm_w.astype(np.float64), eps)
        announce("sweep rmsnorm", m, n, k, head_dim, n_norm)
        out = ops.gemm_fp4_epilogue_rmsnorm_head(*_dev_ops(ac, as_, bc, bs), head_dim, n_norm,
                                                 dev(norm_w, torch.float32) if n_norm else None, eps,
                                                 out_dtype=torch.bfloat16)
        parity.assert_close(host(out), ref, parity.TOL_BF16, group=head_dim,
                            what="rmsnorm hd%d %dx%dx%d" % (head_dim, m, n, k))


@pytest.mark.parametrize("m,n,k", SHAPES, ids=["m%d-n%d-k%d" % s for s in SHAPES])
def test_sweep_swiglu_requant(m, n, k):
    rng = np.random.default_rng(m * 7 + n * 1009 + k)
    operands, h_ref = _swiglu_operands(rng, m, n // 2, k)
    announce("sweep swiglu requant", m, n, k)
    h, mx = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=torch.bfloat16, requant=True)
    parity.assert_close(host(h), h_ref, parity.TOL_BF16, what="swiglu %dx%dx%d" % (m, n, k))
    codes = layout.untile_codes(host(mx.codes), mx.rows, mx.cols)
    scales = layout.untile_scales(host(mx.scales), mx.rows, mx.cols)
    exc, _ = parity.assert_codes_banded(codes, scales, h_ref, "swiglu requant %dx%dx%d" % (m, n, k))
    assert exc <= max(1, 0.001 * h_ref.size)
    # the requant-only launch (no h output) gives the same codes
    _, mx2 = ops.gemm_fp4_epilogue_swiglu(*_dev_ops(*operands), out_dtype=None, requant=True)
    assert np.array_equal(layout.untile_codes(host(mx2.codes), mx2.rows, mx2.cols), codes)
    assert np.array_equal(layout.untile_scales(host(mx2.scales), mx2.rows, mx2.cols), scales)
