"""GPU parity of the MXFP4 quantisation and weight-packing kernels.

Quantising given values has exactly one correct result, so codes and scales
are compared bit for bit with the oracle (bf16 and fp32 inputs, every finite
bf16 value, hand-worked blocks, ragged and empty inputs).
"""

import numpy as np
import pytest
import torch

import golden_io
import layout
import parity
from gpu_util import announce, dev, dev_u8, host
from fp4_diffusion_transformer_amd import ops, workloads
from oracle import gemm as ogemm
from oracle import mxfp4

pytestmark = pytest.mark.gpu


def _quant_both(x64, dtype, lay="rowmajor"):
    """GPU quantisation, returned as row-major packed codes and scales."""
    announce("quantize", x64.shape, dtype, lay)
    mx = ops.quantize_mxfp4(dev(x64, dtype), layout=lay)
    torch.cuda.synchronize()
    rows, cols = x64.shape
    if lay == "tiled":
        return layout.untile_codes(host(mx.codes), rows, cols), layout.untile_scales(host(mx.scales), rows, cols)
    return host(mx.codes), host(mx.scales)


def test_hand_worked_blocks_fp32_and_bf16():
    blocks = golden_io.mxfp4_blocks()
    x = np.array([b[1] for b in blocks])
    for dtype in (torch.float32, torch.bfloat16):
        gc, gs = _quant_both(x, dtype)
        for i, (name, _, scale, packed) in enumerate(blocks):
            assert int(gs[i, 0]) == scale, (name, dtype)
            assert gc[i].tolist() == packed, (name, dtype)


def test_every_bf16_value():
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)].astype(np.float64)
    rows = []
    for d in (0, 1, 2, 3):                     # companions 2**d above each binade
        comp = np.where(vals != 0, np.ldexp(1.0, np.frexp(np.abs(vals))[1] + d), 0.0)
        comp = np.where(np.isfinite(comp) & (comp <= 2.0 ** 127), comp, 0.0)
        blk = np.zeros((len(vals), 32))
        blk[:, 0] = vals
        blk[:, 1] = comp
        rows.append(blk)
    x = np.concatenate(rows)
    x = x[: (len(x) // 8) * 8].reshape(-1, 256)   # 8 blocks per row
    rc, rs = mxfp4.quantize(x)
    gc, gs = _quant_both(x, torch.bfloat16, "tiled")
    parity.assert_codes_exact(gc, gs, rc, rs, "all bf16")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols,lay", [(1, 32, "rowmajor"), (3, 96, "rowmajor"), (257, 3072, "rowmajor"),
                                           (1000, 512, "rowmajor"), (1, 128, "tiled"), (33, 384, "tiled"),
                                           (257, 3072, "tiled")])
def test_random_with_outliers(dtype, rows, cols, lay):
    rng = np.random.default_rng(rows * 7 + cols)
    x = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-30, 30, (rows, 1))
    x[:, rng.choice(cols, max(1, cols // 200), replace=False)] *= 20
    x[0, :7] = [0.0, -0.0, 1e-40, -1e-42, 6.0, -5.0, 0.25]
    x = x.astype(np.float32)
    if dtype == torch.bfloat16:
        x = workloads.to_bf16_values(x)
    x = x.astype(np.float64)
    rc, rs = mxfp4.quantize(x)
    gc, gs = _quant_both(x, dtype, lay)
    parity.assert_codes_exact(gc, gs, rc, rs, "random %s %s" % (dtype, lay))


def test_empty_rows_is_a_no_op():
    x = torch.zeros((0, 128), device="cuda", dtype=torch.bfloat16)
    mx = ops.quantize_mxfp4(x)
    assert mx.rows == 0 and mx.codes.shape == (0, 64) and mx.scales.shape == (0, 4)


def test_workload_activations_bit_exact():
    w = workloads.qkv_hd128(rows=4096)
    rc, rs = mxfp4.quantize(w.x.astype(np.float64))
    gc, gs = _quant_both(w.x.astype(np.float64), torch.bfloat16, "tiled")
    parity.assert_codes_exact(gc, gs, rc, rs, "qkv activations 4096x3072")


def _mx_host(mx):
    if mx.layout == "tiled":
        return (layout.untile_codes(host(mx.codes), mx.rows, mx.cols),
                layout.untile_scales(host(mx.scales), mx.rows, mx.cols))
    return host(mx.codes), host(mx.scales)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lay", ["rowmajor", "tiled"])
def test_pack_weight_plain(dtype, lay):
    rng = np.random.default_rng(5)
    k, n = 512, 320
    w = rng.standard_normal((k, n)).astype(np.float32) / 20
    if dtype == torch.bfloat16:
        w = workloads.to_bf16_values(w)
    announce("pack_weight", k, n, dtype, lay)
    gc, gs = _mx_host(ops.pack_weight(dev(w, dtype), layout=lay))
    rc, rs = mxfp4.quantize(w.astype(np.float64).T)
    parity.assert_codes_exact(gc, gs, rc, rs, "pack plain")


def test_pack_weight_swiglu_interleave():
    rng = np.random.default_rng(6)
    k, n_half = 256, 256
    wg = rng.standard_normal((k, n_half)).astype(np.float32)
    wu = rng.standard_normal((k, n_half)).astype(np.float32) * 3
    g = ops.swiglu_interleave_group()
    announce("pack_weight swiglu", k, 2 * n_half, g)
    gc, gs = _mx_host(ops.pack_weight(dev(np.concatenate([wg, wu], axis=1), torch.float32), interleave_group=g))
    phys = ogemm.interleave_weight(wg, wu, g)
    rc, rs = mxfp4.quantize(phys.astype(np.float64).T)
    parity.assert_codes_exact(gc, gs, rc, rs, "pack interleaved")


@pytest.mark.parametrize("rows,cols", [(1, 64), (1, 96), (5, 160), (7, 512)])
@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_scale_stores_at_any_alignment(rows, cols, offset):
    """The row-major scales buffer needs no alignment (the ABI does not ask
    for any): at every byte offset the kernel must write exactly the
    oracle's bytes and nothing outside the buffer."""
    rng = np.random.default_rng(rows * 13 + cols + offset)
    x = (rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-8, 8, (rows, 1))).astype(np.float32)
    rc, rs = mxfp4.quantize(x.astype(np.float64))
    n = rows * (cols // 32)
    announce("quantize scale stores", rows, cols, offset)
    xd = dev(x, torch.float32)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    buf = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    st = ops.lib().fp4dit_quantize_mxfp4(xd.data_ptr(), ops.F32, rows, cols, codes.data_ptr(),
                                         buf.data_ptr() + 16 + offset, ops.ROWMAJOR,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    b = host(buf)
    parity.assert_codes_exact(host(codes), b[16 + offset:16 + offset + n].reshape(rows, cols // 32), rc, rs,
                              "scales at offset %d" % offset)
    assert (b[:16 + offset] == 0xA5).all() and (b[16 + offset + n:] == 0xA5).all(), "bytes outside the scales"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 128), (31, 128), (33, 640), (95, 384), (1001, 2048), (4101, 1024)])
def test_tiled_stores_stay_inside(dtype, rows, cols):
    """Tiled output with ragged rows: with guard bytes around both tiled
    buffers, the real rows hold the oracle's bytes and nothing is written
    outside the buffers (the padding rows inside them are the library's to
    leave or fill)."""
    rng = np.random.default_rng(rows * 31 + cols)
    x = (rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-12, 12, (rows, 1))).astype(np.float32)
    if dtype == torch.bfloat16:
        x = workloads.to_bf16_values(x)
    x = x.astype(np.float64)
    rc, rs = mxfp4.quantize(x)
    announce("quantize tiled guards", rows, cols, dtype)
    cb = (rows + 1) // 2 * 2 * (cols // 2)
    sb = (rows + 31) // 32 * 32 * (cols // 32)
    g = 256
    cbuf = torch.full((cb + 2 * g,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((sb + 2 * g,), 0xA5, dtype=torch.uint8, device="cuda")
    xd = dev(x, dtype)
    st = ops.lib().fp4dit_quantize_mxfp4(xd.data_ptr(), ops.F32 if dtype == torch.float32 else ops.BF16, rows, cols,
                                         cbuf.data_ptr() + g, sbuf.data_ptr() + g, ops.TILED,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    c, s_ = host(cbuf), host(sbuf)
    parity.assert_codes_exact(layout.untile_codes(c[g:g + cb], rows, cols),
                              layout.untile_scales(s_[g:g + sb], rows, cols), rc, rs, "tiled %dx%d" % (rows, cols))
    assert (c[:g] == 0xA5).all() and (c[g + cb:] == 0xA5).all(), "bytes outside the codes"
    assert (s_[:g] == 0xA5).all() and (s_[g + sb:] == 0xA5).all(), "bytes outside the scales"
