"""GPU parity of the unfused epilogue kernels (per-head RMSNorm and SwiGLU
as launches of their own over a bf16 GEMM output) against the oracle, and
of the unfused chain GEMM -> bf16 -> epilogue at a full DiT-1K shape."""

import numpy as np
import pytest
import torch

import layout
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


@pytest.mark.parametrize("make", [workloads.qkv_hd128, workloads.qkv_hd256], ids=["hd128", "hd256"])
def test_unfused_chain_qkv_full_size(make):
    """quantise -> GEMM (bf16 store) -> RMSNorm launch, at the QKV shapes
    (4096 x 9216 x 3072 with hd 128, 4096 x 12288 x 4096 with hd 256);
    sampled rows against the oracle's RMSNorm of the bf16-rounded GEMM
    output."""
    wl = make()
    announce("unfused chain", wl.name, wl.m, wl.n, wl.k)
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


def test_unfused_chain_ffn_up_full_size():
    """quantise -> GEMM over the interleaved [gate | up] weight (bf16 store)
    -> SwiGLU launch -> quantise, at the FFN-up shape (4096 x 24576 x 3072).
    Sampled rows: h against the oracle's SwiGLU of the bf16-rounded gate and
    up outputs, and the MXFP4 codes of h within the rounding band of that
    reference (h itself is a bf16 rounding of it)."""
    wl = workloads.ffn_up_swiglu(requant=False)
    g = ops.swiglu_interleave_group()
    n_half = wl.w_gate.shape[1]
    announce("unfused chain ffn_up", wl.m, 2 * n_half, wl.k)
    a = ops.quantize_mxfp4(dev(wl.x, torch.bfloat16))
    b = ops.pack_weight(dev(np.concatenate([wl.w_gate, wl.w_up], axis=1), torch.float32), g)
    c = ops.gemm_fp4_epilogue_none(a, b, out_dtype=torch.bfloat16)
    h = ops.swiglu(c, g)
    hq = ops.quantize_mxfp4(h)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.m - 1], np.random.default_rng(6).choice(wl.m, 14, replace=False)]))
    ac, as_ = mxfp4.quantize(wl.x[rows].astype(np.float64))
    gc_, gs_ = mxfp4.quantize(wl.w_gate.astype(np.float64).T)
    uc_, us_ = mxfp4.quantize(wl.w_up.astype(np.float64).T)
    g_ref = obf16.round_bf16(ogemm.gemm(ac, as_, gc_, gs_))
    u_ref = obf16.round_bf16(ogemm.gemm(ac, as_, uc_, us_))
    h_ref = ogemm.swiglu(g_ref, u_ref)
    parity.assert_close(host(h)[rows], h_ref, parity.TOL_BF16, what="unfused swiglu chain")
    codes = layout.untile_codes(host(hq.codes), wl.m, n_half)[rows]
    scales = layout.untile_scales(host(hq.scales), wl.m, n_half)[rows]
    # Per-element band from the oracle: the GPU's gate and up are bf16
    # roundings of fp32 sums, which may land on the neighbouring bf16 value
    # of the oracle's rounding (one ulp), and h itself is rounded to bf16
    # (half an ulp, taken as 2^-8 |h| with margin).  With h = silu(g) u:
    #   |dh| <= |u silu'(g)| ulp(g) + |silu(g)| ulp(u) + 2^-8 |h|,
    # silu'(g) = s (1 + g (1 - s)), s = sigmoid(g); in scaled units that is
    # the code band, and its block maximum over the block amax the scale band.
    def ulp_bf16(v):
        e = np.frexp(np.abs(v))[1]
        return np.where(v == 0, 2.0 ** -133, 2.0 ** (e - 8.0))

    sg = 1.0 / (1.0 + np.exp(-g_ref))
    dh = (np.abs(u_ref * sg * (1.0 + g_ref * (1.0 - sg))) * ulp_bf16(g_ref)
          + np.abs(g_ref * sg) * ulp_bf16(u_ref) + 2.0 ** -8 * np.abs(h_ref))
    ref = mxfp4.quantize(h_ref, return_scaled=True)
    shared = np.repeat(ref[1].astype(np.float64) - 127.0, 32, axis=1)
    m_, n_ = h_ref.shape
    blk_amax = np.max(np.abs(h_ref).reshape(m_, n_ // 32, 32), axis=2)
    blk_dh = np.max(dh.reshape(m_, n_ // 32, 32), axis=2)
    exc, _ = parity.assert_codes_banded(codes, scales, h_ref, "unfused swiglu chain codes", ref=ref,
                                        tau=dh / 2.0 ** shared + parity.TAU,
                                        amax_rel=blk_dh / np.maximum(blk_amax, 1e-300) + parity.AMAX_REL)
    assert exc <= 0.02 * h_ref.size
