"""GPU check of fp4dit_mx_relayout: a byte permutation between the row-major
MXFP4 layout and the GEMM's tiled layout, so it must equal the layout
definition (tests/layout.py, written from include/fp4dit.h) byte for byte,
padding rows included, and round-trip exactly."""

import numpy as np
import pytest
import torch

import layout
from gpu_util import announce, dev, dev_u8, host
from fp4_diffusion_transformer_amd import ops

pytestmark = pytest.mark.gpu


def _random_mx(rng, rows, cols):
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, cols // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("rows,cols", [(1, 128), (33, 256), (300, 512), (64, 3072), (257, 384)])
def test_rowmajor_to_tiled_and_back(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    codes, scales = _random_mx(rng, rows, cols)
    announce("relayout", rows, cols)
    rm = ops.MxTensor(dev_u8(codes), dev_u8(scales), rows, cols, "rowmajor")
    ti = ops.mx_relayout(rm, "tiled")
    torch.cuda.synchronize()
    assert np.array_equal(host(ti.codes), layout.tile_codes(codes))           # padding rows are zero
    assert np.array_equal(host(ti.scales), layout.tile_scales(scales))
    back = ops.mx_relayout(ti, "rowmajor")
    torch.cuda.synchronize()
    assert np.array_equal(host(back.codes), codes) and np.array_equal(host(back.scales), scales)
    # same layout on both sides: a copy, whose tiled padding bytes come out
    # as zero whatever the input's padding held
    pad_c = layout.tile_codes(np.ones_like(codes)) == 0
    pad_s = layout.tile_scales(np.ones_like(scales)) == 0
    dirty_c, dirty_s = layout.tile_codes(codes), layout.tile_scales(scales)
    dirty_c[pad_c] = 0x5A
    dirty_s[pad_s] = 0x5A
    ti2 = ops.mx_relayout(ops.MxTensor(dev_u8(dirty_c), dev_u8(dirty_s), rows, cols, "tiled"), "tiled")
    rm2 = ops.mx_relayout(rm, "rowmajor")
    torch.cuda.synchronize()
    assert np.array_equal(host(ti2.codes), host(ti.codes)) and np.array_equal(host(ti2.scales), host(ti.scales))
    assert np.array_equal(host(rm2.codes), codes) and np.array_equal(host(rm2.scales), scales)


def test_rowmajor_copy_cols_multiple_of_32():
    rng = np.random.default_rng(5)
    codes, scales = _random_mx(rng, 17, 96)
    announce("relayout rowmajor copy", 17, 96)
    out = ops.mx_relayout(ops.MxTensor(dev_u8(codes), dev_u8(scales), 17, 96, "rowmajor"), "rowmajor")
    torch.cuda.synchronize()
    assert np.array_equal(host(out.codes), codes) and np.array_equal(host(out.scales), scales)


def test_quantize_rowmajor_relayout_feeds_the_gemm():
    """A caller with plain row-major MXFP4 reaches the GEMM through the
    relayout: the output equals the one from the tiled quantiser bit for bit."""
    rng = np.random.default_rng(6)
    m, n, k = 300, 512, 768
    x = dev(rng.standard_normal((m, k)).astype(np.float32), torch.bfloat16)
    w = dev((rng.standard_normal((k, n)) / np.sqrt(k)).astype(np.float32), torch.float32)
    announce("relayout into gemm", m, n, k)
    b = ops.pack_weight(w)
    a_direct = ops.quantize_mxfp4(x, layout="tiled")
    a_via = ops.mx_relayout(ops.quantize_mxfp4(x, layout="rowmajor"), "tiled")
    out1 = ops.gemm_fp4_epilogue_none(a_direct, b, out_dtype=torch.float32)
    out2 = ops.gemm_fp4_epilogue_none(a_via, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
