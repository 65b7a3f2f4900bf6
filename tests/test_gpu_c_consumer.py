"""The C ABI from C: tests/c_consumer.c (C99, built with the library) creates
its own stream and buffers and runs quantise -> weight pack -> FP4 GEMM with
the per-head RMSNorm epilogue through include/fp4dit.h; its output is
checked against the oracle.  Ragged M, four hd-128 heads."""

import os
import subprocess

import numpy as np
import pytest

import parity
from gpu_util import announce
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
