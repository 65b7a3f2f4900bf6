"""The seeded input generators are deterministic and follow their recipe."""

import numpy as np

from fp4_diffusion_transformer_amd import workloads


def test_deterministic():
    a = workloads.qkv_hd128(rows=64)
    b = workloads.qkv_hd128(rows=64)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w[:, :64], b.w[:, :64])


def test_bf16_values_and_outliers():
    w = workloads.qkv_hd128(rows=256)
    u = w.x.view(np.uint32)
    assert not (u & 0xFFFF).any()                       # exactly bf16
    col_rms = np.sqrt(np.mean(w.x.astype(np.float64) ** 2, axis=0))
    assert (col_rms > 10).sum() == 15                   # round(0.005 * 3072) outlier channels
    assert w.norm_w.shape == (6144,)
    assert np.array_equal(w.norm_w[:128], w.norm_w[128:256])


def test_transforms_conditioned():
    t = workloads.transforms(99, 4)
    assert not (t.view(np.uint32) & 0xFFFF).any()
    for b in range(4):
        assert np.linalg.cond(t[b].astype(np.float64)) < 10
