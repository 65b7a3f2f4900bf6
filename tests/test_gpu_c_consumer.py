"""The C ABI from C: tests/c_consumer.c (C99, built with the library) creates
its own stream and buffers and runs quantise -> weight pack -> FP4 GEMM with
the per-head RMSNorm epilogue (ragged M, four hd-128 heads), or the SwiGLU
epilogue with MXFP4 requantisation, through include/fp4dit.h; its output is
checked against the oracle."""

import os
import subprocess

import numpy as np
import pytest

import parity
from gpu_util import announce
import layout
from oracle import bf16 as obf16
from oracle import gemm as ogemm
from oracle import mxfp4

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_consumer")


def test_c_program_runs_the_rmsnorm_gemm(tmp_path):
    if not os.path.exists(BIN):
        pytest.fail("tests/c_consumer is not built (python -m fp4_diffusion_transformer_amd.build)")
    m, n, k = 300, 512, 512
    rng = np.random.default_rng(77)
    x = obf16.round_bf16(rng.standard_normal((m, k)))                 # exact bf16 values
    w = (rng.standard_normal((k, n)) / np.sqrt(k)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).tofile(tmp_path / "x.bin")
    w.tofile(tmp_path / "w.bin")
    g.tofile(tmp_path / "g.bin")
    announce("c consumer", m, n, k)
    r = subprocess.run([BIN, str(tmp_path), str(m), str(n), str(k)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    y = (np.fromfile(tmp_path / "y.bin", dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    y = y.reshape(m, n).astype(np.float64)
    ac, as_ = mxfp4.quantize(x.astype(np.float64))
    bc, bs = mxfp4.quantize(w.astype(np.float64).T)
    ref = ogemm.rmsnorm_head(ogemm.gemm(ac, as_, bc, bs), 128, n, g.astype(np.float64), 1e-6)
    parity.assert_close(y, ref, parity.TOL_BF16, group=128, what="C consumer")


def test_c_program_runs_the_swiglu_requant_gemm(tmp_path):
    """The SwiGLU GEMM with MXFP4 requantisation from C: the program packs
    [gate | up] with the library's interleave group and writes tiled codes
    and scales, compared with the oracle's SwiGLU within the rounding band."""
    if not os.path.exists(BIN):
        pytest.fail("tests/c_consumer is not built (python -m fp4_diffusion_transformer_amd.build)")
    m, nh, k = 300, 256, 512
    rng = np.random.default_rng(78)
    x = obf16.round_bf16(rng.standard_normal((m, k)))
    w = (rng.standard_normal((k, 2 * nh)) / np.sqrt(k)).astype(np.float32)       # [gate | up]
    (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).tofile(tmp_path / "x.bin")
    w.tofile(tmp_path / "w.bin")
    announce("c consumer swiglu", m, 2 * nh, k)
    r = subprocess.run([BIN, str(tmp_path), str(m), str(2 * nh), str(k), "swiglu"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    codes = layout.untile_codes(np.fromfile(tmp_path / "codes.bin", dtype=np.uint8), m, nh)
    scales = layout.untile_scales(np.fromfile(tmp_path / "scales.bin", dtype=np.uint8), m, nh)
    ac, as_ = mxfp4.quantize(x.astype(np.float64))
    gc_, gs_ = mxfp4.quantize(w[:, :nh].astype(np.float64).T)
    uc_, us_ = mxfp4.quantize(w[:, nh:].astype(np.float64).T)
    h_ref = ogemm.swiglu(ogemm.gemm(ac, as_, gc_, gs_), ogemm.gemm(ac, as_, uc_, us_))
    exc, _ = parity.assert_codes_banded(codes, scales, h_ref, "C consumer swiglu requant")
    assert exc <= 0.001 * h_ref.size
