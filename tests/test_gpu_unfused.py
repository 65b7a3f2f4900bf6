"""GPU parity of the unfused epilogue kernels (per-head RMSNorm and SwiGLU
as launches of their own over a bf16 GEMM output) against the oracle, and
of the unfused chain GEMM -> bf16 -> epilogue at a full DiT-1K shape."""

import numpy as np
import pytest
import torch

import parity
from gpu_util import announce, dev, host
from fp4_diffusion_transformer_amd import ops, workloads
from oracle import bf16 as obf16
from oracle import gemm as ogemm
from oracle import mxfp4

pytestmark = pytest.mark.gpu


def _bf16_input(rng, rows, cols):
    x = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-6, 7, (rows, 1))
    x[rng.choice(rows, min(rows, 3), replace=False)] *= 1e-4      # heads where eps matters
    return obf16.round_bf16(x)                                     # exact bf16 values


@pytest.mark.parametrize("rows,cols,hd,n_norm", [(333, 1024, 128, 768), (64, 1536, 256, 1024),
                                                 (1, 256, 128, 256), (7, 512, 256, 0)])
def test_rmsnorm_head(rows, cols, hd, n_norm):
    rng = np.random.default_rng(rows + cols + hd)
    x = _bf16_input(rng, rows, cols)
    w = rng.uniform(0.5, 1.5, n_norm).astype(np.float32)
    eps = 1e-6
    ref = ogemm.rmsnorm_head(x, hd, n_norm, w.astype(np.float64), eps)
    announce("unfused rmsnorm", rows, cols, hd, n_norm)
    out = ops.rmsnorm_head(dev(x, torch.bfloat16), hd, n_norm, dev(w, torch.float32) if n_norm else None, eps)
    parity.assert_close(host(out), ref, parity.TOL_BF16, group=hd, what="unfused rmsnorm")
    # pass-through columns are copied bit for bit
    assert np.array_equal(host(out)[:, n_norm:], x[:, n_norm:])


def test_rmsnorm_head_in_place():
    rng = np.random.default_rng(3)
    x = _bf16_input(rng, 100, 768)
    w = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    ref = ogemm.rmsnorm_head(x, 256, 512, w.astype(np.float64), 1e-6)
    announce("unfused rmsnorm in place")
    xd = dev(x, torch.bfloat16)
    out = ops.rmsnorm_head(xd, 256, 512, dev(w, torch.float32), 1e-6, out=xd)
    assert out is xd
    parity.assert_close(host(xd), ref, parity.TOL_BF16, group=256, what="unfused rmsnorm in place")


@pytest.mark.parametrize("rows,n_half,g", [(300, 512, 32), (5, 96, 8), (1, 256, 32)])
def test_swiglu(rows, n_half, g):
    rng = np.random.default_rng(rows + n_half + g)
    c = obf16.round_bf16(rng.standard_normal((rows, 2 * n_half)) * 4)
    ref = ogemm.swiglu_from_interleaved(c, g)
    announce("unfused swiglu", rows, n_half, g)
    h = ops.swiglu(dev(c, torch.bfloat16), g)
    parity.assert_close(host(h), ref, parity.TOL_BF16, what="unfused swiglu")


def test_unfused_chain_qkv_hd128_full_size():
    """quantise -> GEMM (bf16 store) -> RMSNorm launch, at the QKV hd128
    shape (4096 x 9216 x 3072); sampled rows against the oracle's RMSNorm of
    the bf16-rounded GEMM output."""
    wl = workloads.qkv_hd128()
    announce("unfused chain qkv_hd128", wl.m, wl.n, wl.k)
    a = ops.quantize_mxfp4(dev(wl.x, torch.bfloat16))
    b = ops.pack_weight(dev(wl.w, torch.float32))
    c = ops.gemm_fp4_epilogue_none(a, b, out_dtype=torch.bfloat16)
    y = ops.rmsnorm_head(c, wl.head_dim, wl.n_norm, dev(wl.norm_w, torch.float32), wl.eps)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.m - 1], np.random.default_rng(4).choice(wl.m, 16, replace=False)]))
    ac, as_ = mxfp4.quantize(wl.x[rows].astype(np.float64))
    bc, bs = mxfp4.quantize(wl.w.astype(np.float64).T)
    c_ref = obf16.round_bf16(ogemm.gemm(ac, as_, bc, bs))
    ref = ogemm.rmsnorm_head(c_ref, wl.head_dim, wl.n_norm, wl.norm_w.astype(np.float64), wl.eps)
    parity.assert_close(host(y)[rows], ref, parity.TOL_BF16, group=wl.head_dim, what="unfused chain")
