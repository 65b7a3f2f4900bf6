"""End-to-end GPU parity on the full-size DiT workloads.

The GPU runs every workload at its full size, in the launch configuration
the benchmark times (tiled operands, bf16 / MXFP4 outputs).  Rows are
independent, so the oracle recomputes a seeded sample of rows (first, last,
random) from the same inputs; activation codes are compared in full.  The
tiny workload is compared in full.
"""

import functools

import numpy as np
import pytest
import torch

import layout
import parity
from gpu_util import announce, dev, host
from fp4_diffusion_transformer_amd import ops, workloads
from oracle import gemm as ogemm
from oracle import mxfp4, transform

pytestmark = pytest.mark.gpu


_dit_block = functools.lru_cache(maxsize=1)(workloads.dit_block)


def _rows(m, n=24, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, m - 1], rng.choice(m, n, replace=False)]))


def _untile(mx):
    return (layout.untile_codes(host(mx.codes), mx.rows, mx.cols),
            layout.untile_scales(host(mx.scales), mx.rows, mx.cols))


def _gpu_linear(wl, x_dev=None):
    """The benchmark's fused linear: quantise (or transform + quantise) the
    activations, pack the weight, fused GEMM + epilogue.  Returns
    (activation MxTensor, weight MxTensor, output(s))."""
    if x_dev is None:
        x_dev = dev(wl.x, torch.bfloat16 if wl.x_bf16 else torch.float32)
    t_dev = None if wl.t is None else dev(wl.t, torch.bfloat16)
    if t_dev is None:
        a = ops.quantize_mxfp4(x_dev)
    else:
        _, a = ops.block_transform(x_dev, t_dev, quantize=True)
    if wl.epilogue == "swiglu":
        w = dev(np.concatenate([wl.w_gate, wl.w_up], axis=1), torch.float32)
        group = ops.swiglu_interleave_group()
    else:
        w = dev(wl.w, torch.float32)
        group = 0
    if t_dev is not None:
        w = ops.fold_inverse_transform(w, t_dev)
    b = ops.pack_weight(w, interleave_group=group)
    del w
    if wl.epilogue == "rmsnorm_head":
        out = ops.gemm_fp4_epilogue_rmsnorm_head(a, b, wl.head_dim, wl.n_norm, dev(wl.norm_w, torch.float32),
                                                 wl.eps, out_dtype=torch.bfloat16)
    elif wl.epilogue == "swiglu":
        out = ops.gemm_fp4_epilogue_swiglu(a, b, out_dtype=None if wl.requant else torch.bfloat16,
                                           requant=wl.requant)
    else:
        out = ops.gemm_fp4_epilogue_none(a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    return a, b, out


def _oracle_linear(wl, x_rows, w_codes=None):
    """Oracle output rows for the activations x_rows (float64)."""
    t = None if wl.t is None else wl.t.astype(np.float64)
    ac, as_ = mxfp4.quantize(x_rows) if t is None else transform.transform_quantize(x_rows, t)
    if wl.epilogue == "swiglu":
        wg, wu = wl.w_gate.astype(np.float64), wl.w_up.astype(np.float64)
        if t is not None:
            wg, wu = transform.fold_inverse(wg, t), transform.fold_inverse(wu, t)
        gc_, gs_ = mxfp4.quantize(wg.T)
        uc_, us_ = mxfp4.quantize(wu.T)
        return ogemm.swiglu(ogemm.gemm(ac, as_, gc_, gs_), ogemm.gemm(ac, as_, uc_, us_))
    w = wl.w.astype(np.float64)
    if t is not None:
        w = transform.fold_inverse(w, t)
    bc, bs = mxfp4.quantize(w.T)
    c = ogemm.gemm(ac, as_, bc, bs)
    if wl.epilogue == "rmsnorm_head":
        return ogemm.rmsnorm_head(c, wl.head_dim, wl.n_norm, wl.norm_w.astype(np.float64), wl.eps)
    return c


def test_tiny_full_compare():
    wl = workloads.tiny()
    announce("config tiny", wl.m, wl.n, wl.k)
    a, b, out = _gpu_linear(wl)
    ac, as_ = mxfp4.quantize(wl.x.astype(np.float64))
    parity.assert_codes_exact(*_untile(a), ac, as_, "tiny activations")
    ref = _oracle_linear(wl, wl.x.astype(np.float64))
    parity.assert_close(host(out), ref, parity.TOL_BF16, group=wl.head_dim, what="tiny rmsnorm")


@pytest.mark.parametrize("name", ["qkv_hd128", "qkv_hd256"])
def test_qkv_full_size(name):
    wl = getattr(workloads, name)()
    announce("config", name, wl.m, wl.n, wl.k)
    a, b, out = _gpu_linear(wl)
    x64 = wl.x.astype(np.float64)
    ac, as_ = mxfp4.quantize(x64)
    parity.assert_codes_exact(*_untile(a), ac, as_, name + " activations")
    rows = _rows(wl.m)
    ref = _oracle_linear(wl, x64[rows])
    parity.assert_close(host(out)[rows], ref, parity.TOL_BF16, group=wl.head_dim, what=name)


def test_ffn_up_swiglu_requant_full_size():
    wl = workloads.ffn_up_swiglu(requant=True)
    announce("config ffn_up", wl.m, wl.n, wl.k)
    a, b, (h, mx) = _gpu_linear(wl)
    rows = _rows(wl.m, seed=4)
    ref = _oracle_linear(wl, wl.x.astype(np.float64)[rows])
    codes, scales = _untile(mx)
    exc, blk = parity.assert_codes_banded(codes[rows], scales[rows], ref, "ffn up requant")
    assert exc <= 0.001 * ref.size


def _mx_dev(codes, scales):
    """Oracle codes (unpacked, row-major) -> tiled MxTensor on the device."""
    rows, cols = codes.shape
    return ops.MxTensor(dev(layout.tile_codes(mxfp4.pack_codes(codes)), torch.uint8),
                        dev(layout.tile_scales(scales), torch.uint8), rows, cols, "tiled")


@pytest.mark.parametrize("stage", ["qkv", "up", "down"])
def test_dit_block_batch4_stages(stage):
    """Batch of 4 images with the block transform, stage by stage.

    The transform is summed in fp32 on the GPU and in float64 by the oracle
    (and the weight fold is rounded to fp32 before packing), so a few codes
    whose value sits on a rounding midpoint may legitimately differ; a single
    such code moves a whole output row, so the chain is not compared end to
    end.  Instead: (1) activation transform + quantise codes, all 16384 rows,
    and (2) folded weight codes, against the oracle with the midpoint band;
    (3) the fused GEMM + epilogue on the oracle's own operand codes, sampled
    rows.  The down layer runs on its seeded stand-in input."""
    wl = dict(zip(["qkv", "up", "down"], _dit_block()))[stage]
    t64 = wl.t.astype(np.float64)
    announce("config dit_block", stage, wl.m, wl.n, wl.k)
    x_dev = dev(wl.x, torch.bfloat16)
    t_dev = dev(wl.t, torch.bfloat16)
    _, a = ops.block_transform(x_dev, t_dev, quantize=True)            # full size, as benchmarked
    torch.cuda.synchronize()
    # (1) activation codes on the first 4096 rows (rows are independent)
    n_chk = 4096
    y_ref = transform.block_transform(wl.x[:n_chk].astype(np.float64), t64)
    gc, gs = _untile(a)
    exc, blk = parity.assert_codes_banded(gc[:n_chk], gs[:n_chk], y_ref, "dit %s activations" % stage)
    assert exc <= 1e-4 * y_ref.size
    del a, y_ref, gc, gs
    # (2) weights: fold T^-1 into W on the GPU, pack, compare codes
    if wl.epilogue == "swiglu":
        w = np.concatenate([wl.w_gate, wl.w_up], axis=1)
        group = ops.swiglu_interleave_group()
        pair, is_up = ogemm.interleave_columns(wl.w_gate.shape[1], group)
        src = np.where(is_up, pair + wl.w_gate.shape[1], pair)        # physical -> logical column
    else:
        w, group, src = wl.w, 0, np.arange(wl.w.shape[1])
    b = ops.pack_weight(ops.fold_inverse_transform(dev(w, torch.float32), t_dev), interleave_group=group)
    torch.cuda.synchronize()
    w_fold = transform.fold_inverse(w.astype(np.float64), t64)[:, src]  # physical column order
    exc, blk = parity.assert_codes_banded(*_untile(b), w_fold.T, "dit %s weights" % stage)
    assert exc <= 1e-4 * w_fold.size
    del b
    # (3) fused GEMM + epilogue at full size on the oracle's own operand codes
    ac, as_ = transform.transform_quantize(wl.x.astype(np.float64), t64)
    bc, bs = mxfp4.quantize(w_fold.T)
    del w_fold
    a_dev, b_dev = _mx_dev(ac, as_), _mx_dev(bc, bs)
    rows = _rows(wl.m, n=16, seed=5)
    c = ogemm.gemm(ac[rows], as_[rows], bc, bs)
    del ac, as_
    if stage == "qkv":
        out = ops.gemm_fp4_epilogue_rmsnorm_head(a_dev, b_dev, wl.head_dim, wl.n_norm,
                                                 dev(wl.norm_w, torch.float32), wl.eps)
        ref = ogemm.rmsnorm_head(c, wl.head_dim, wl.n_norm, wl.norm_w.astype(np.float64), wl.eps)
        group_cols = wl.head_dim
    elif stage == "up":
        out, _ = ops.gemm_fp4_epilogue_swiglu(a_dev, b_dev, out_dtype=torch.bfloat16)
        ref = ogemm.swiglu_from_interleaved(c, group)
        group_cols = None
    else:
        out = ops.gemm_fp4_epilogue_none(a_dev, b_dev)
        ref, group_cols = c, None
    torch.cuda.synchronize()
    parity.assert_close(host(out)[rows], ref, parity.TOL_BF16, group=group_cols, what="dit " + stage)


def test_dit_block_up_fused_down_transform():
    """The batch-4 block's FFN-up GEMM with SwiGLU, the down layer's block
    transform (384 matrices) and MXFP4 fused in its epilogue, at full size
    (16384 x 24576 x 3072) on the oracle's operand codes; sampled rows
    against the oracle's SwiGLU -> transform -> quantise."""
    _, up, down = _dit_block()
    t_up = up.t.astype(np.float64)
    announce("config dit_block up fused with the down transform", up.m, up.n, up.k)
    ac, as_ = transform.transform_quantize(up.x.astype(np.float64), t_up)
    wg = transform.fold_inverse(up.w_gate.astype(np.float64), t_up)
    wu = transform.fold_inverse(up.w_up.astype(np.float64), t_up)
    gc_, gs_ = mxfp4.quantize(wg.T)
    uc_, us_ = mxfp4.quantize(wu.T)
    del wg, wu
    pair, is_up = ogemm.interleave_columns(gc_.shape[0], ops.swiglu_interleave_group())
    bc = np.where(is_up[:, None], uc_[pair], gc_[pair])
    bs = np.where(is_up[:, None], us_[pair], gs_[pair])
    rows = _rows(up.m, n=16, seed=7)
    c_g = ogemm.gemm(ac[rows], as_[rows], gc_, gs_)
    c_u = ogemm.gemm(ac[rows], as_[rows], uc_, us_)
    a_dev, b_dev = _mx_dev(ac, as_), _mx_dev(bc, bs)
    del ac, as_, bc, bs
    _, mx = ops.gemm_fp4_epilogue_swiglu_transform(a_dev, b_dev, dev(down.t, torch.bfloat16))
    torch.cuda.synchronize()
    codes, scales = _untile(mx)
    parity.assert_fused_codes(codes[rows], scales[rows], c_g, c_u, down.t, "dit up fused down transform")


# ----------------------------------------------------------------------------
# The batch-4 block chained on the GPU exactly as the benchmark runs it.

def _gpu_weight(w, t_dev, group):
    """The benchmark's weight preparation on the GPU: fold T^-1, pack (tiled)."""
    return ops.pack_weight(ops.fold_inverse_transform(dev(w, torch.float32), t_dev), interleave_group=group)


def _oracle_weight_codes(w, t64, src):
    """Oracle codes of the folded weight in physical column order [N, K]."""
    w_fold = transform.fold_inverse(w.astype(np.float64), t64)[:, src]
    return mxfp4.quantize(w_fold.T)


def _equal_rows(gpu_mx, ref_codes, ref_scales, rows):
    """Rows (of `rows`) whose GPU codes and scales equal the oracle's."""
    gc, gs = _untile(gpu_mx)
    gc, gs = gc[rows], gs[rows]
    return np.all(gc == mxfp4.pack_codes(ref_codes), axis=1) & np.all(gs == ref_scales, axis=1)


def _equal_weight_rows(gpu_mx, bc, bs):
    """Physical output columns whose GPU weight codes and scales (all of K)
    equal the oracle's."""
    gc, gs = _untile(gpu_mx)
    return np.all(gc == mxfp4.pack_codes(bc), axis=1) & np.all(gs == bs, axis=1)


@pytest.mark.parametrize("stage", ["qkv", "up", "down"])
def test_dit_block_batch4_chain(stage):
    """Each stage of the batch-4 block chained on the GPU as the benchmark
    runs it -- block transform + quantise of the activations, T^-1 folded
    into the weight and packed, fused GEMM + epilogue, all on the device --
    against the oracle run from the same inputs (x, W, T, gains) on sampled
    rows.  The transform and the fold are fp32 sums on the GPU, so a code on
    a rounding midpoint may differ (within the S13 band, checked by the stage
    test above); where one does, the whole row (activations) or output
    column (weights) legitimately differs, so those are left out and
    counted, and everything else must meet the plain tolerance."""
    wl = dict(zip(["qkv", "up", "down"], _dit_block()))[stage]
    t64 = wl.t.astype(np.float64)
    announce("config dit_block chain", stage, wl.m, wl.n, wl.k)
    t_dev = dev(wl.t, torch.bfloat16)
    _, a = ops.block_transform(dev(wl.x, torch.bfloat16), t_dev, quantize=True)
    if wl.epilogue == "swiglu":
        w = np.concatenate([wl.w_gate, wl.w_up], axis=1)
        group = ops.swiglu_interleave_group()
        pair, is_up = ogemm.interleave_columns(wl.w_gate.shape[1], group)
        src = np.where(is_up, pair + wl.w_gate.shape[1], pair)
    else:
        w, group, src = wl.w, 0, np.arange(wl.w.shape[1])
    b = _gpu_weight(w, t_dev, group)
    if stage == "qkv":
        out = ops.gemm_fp4_epilogue_rmsnorm_head(a, b, wl.head_dim, wl.n_norm, dev(wl.norm_w, torch.float32),
                                                 wl.eps)
    elif stage == "up":
        out, _ = ops.gemm_fp4_epilogue_swiglu(a, b, out_dtype=torch.bfloat16)
    else:
        out = ops.gemm_fp4_epilogue_none(a, b)
    torch.cuda.synchronize()
    rows = _rows(wl.m, n=24, seed=11)
    ac, as_ = transform.transform_quantize(wl.x[rows].astype(np.float64), t64)
    keep_r = _equal_rows(a, ac, as_, rows)
    bc, bs = _oracle_weight_codes(w, t64, src)
    keep_c = _equal_weight_rows(b, bc, bs)                        # per physical column
    c = ogemm.gemm(ac[keep_r], as_[keep_r], bc, bs)
    got = host(out)[rows[keep_r]]
    if stage == "qkv":
        ref = ogemm.rmsnorm_head(c, wl.head_dim, wl.n_norm, wl.norm_w.astype(np.float64), wl.eps)
        # a normalised head depends on all of its columns
        heads = keep_c[:wl.n_norm].reshape(-1, wl.head_dim).all(axis=1)
        col_ok = np.concatenate([np.repeat(heads, wl.head_dim), keep_c[wl.n_norm:]])
        group_cols = wl.head_dim
    elif stage == "up":
        ref = ogemm.swiglu_from_interleaved(c, group)
        # output j comes from its gate and its up column
        n_half = wl.w_gate.shape[1]
        ok_logical = np.zeros(2 * n_half, dtype=bool)
        ok_logical[src] = keep_c
        col_ok = ok_logical[:n_half] & ok_logical[n_half:]
        group_cols = None
    else:
        ref, col_ok, group_cols = c, keep_c, None
    n_rows, n_cols = int(keep_r.sum()), int(col_ok.sum())
    print("[chain %s] rows compared %d of %d (%d left out: an activation code on a midpoint); output columns "
          "compared %d of %d (%d left out: a folded-weight code on a midpoint)"
          % (stage, n_rows, len(rows), len(rows) - n_rows, n_cols, col_ok.size, col_ok.size - n_cols), flush=True)
    assert n_rows >= len(rows) // 2 and n_cols >= 0.9 * col_ok.size, "too many codes on midpoints"
    mask = np.broadcast_to(col_ok, ref.shape)
    parity.assert_close(got, ref, parity.TOL_BF16, group=group_cols, what="dit chain " + stage, mask=mask)


def test_dit_block_batch4_fused_chain():
    """The benchmark's fused batch-4 block from the FFN-up input to the down
    projection's output, entirely on the GPU: up-input transform + quantise,
    FFN-up GEMM with SwiGLU -> the down layer's 384 block transforms -> MXFP4
    in its epilogue, then the down GEMM (weights folded and packed on the
    GPU) -- against the oracle's SwiGLU -> transform -> quantise -> down GEMM
    from the same inputs.  Rows are compared where the GPU's up activations
    and its fused down activations both equal the oracle's codes (else a code
    on a midpoint changed the row; counted), and output columns where the
    down weight codes equal the oracle's."""
    _, up, down = _dit_block()
    t_up, t_dn = up.t.astype(np.float64), down.t.astype(np.float64)
    announce("config dit_block fused chain", up.m, up.n, up.k, down.n)
    _, a_up = ops.block_transform(dev(up.x, torch.bfloat16), dev(up.t, torch.bfloat16), quantize=True)
    group = ops.swiglu_interleave_group()
    w_up = np.concatenate([up.w_gate, up.w_up], axis=1)
    b_up = _gpu_weight(w_up, dev(up.t, torch.bfloat16), group)
    _, a_dn = ops.gemm_fp4_epilogue_swiglu_transform(a_up, b_up, dev(down.t, torch.bfloat16))
    b_dn = _gpu_weight(down.w, dev(down.t, torch.bfloat16), 0)
    out = ops.gemm_fp4_epilogue_none(a_dn, b_dn)
    torch.cuda.synchronize()
    del b_up
    rows = _rows(up.m, n=24, seed=13)
    ac, as_ = transform.transform_quantize(up.x[rows].astype(np.float64), t_up)
    keep_up = _equal_rows(a_up, ac, as_, rows)
    wg = transform.fold_inverse(up.w_gate.astype(np.float64), t_up)
    wu = transform.fold_inverse(up.w_up.astype(np.float64), t_up)
    gc_, gs_ = mxfp4.quantize(wg.T)
    uc_, us_ = mxfp4.quantize(wu.T)
    del wg, wu
    c_g = ogemm.gemm(ac, as_, gc_, gs_)
    c_u = ogemm.gemm(ac, as_, uc_, us_)
    dc, ds = ogemm.swiglu_transform_requantize(c_g, c_u, t_dn)
    keep_dn = _equal_rows(a_dn, dc, ds, rows)
    keep_r = keep_up & keep_dn
    bc, bs = _oracle_weight_codes(down.w, t_dn, np.arange(down.w.shape[1]))
    keep_c = _equal_weight_rows(b_dn, bc, bs)
    ref = ogemm.gemm(dc[keep_r], ds[keep_r], bc, bs)
    got = host(out)[rows[keep_r]]
    n_rows, n_cols = int(keep_r.sum()), int(keep_c.sum())
    print("[fused chain] rows compared %d of %d (up activations differ in %d, fused down activations in %d); "
          "output columns compared %d of %d" % (n_rows, len(rows), int((~keep_up).sum()), int((~keep_dn).sum()),
                                                 n_cols, keep_c.size), flush=True)
    assert n_rows >= len(rows) // 2 and n_cols >= 0.9 * keep_c.size, "too many codes on midpoints"
    parity.assert_close(got, ref, parity.TOL_BF16, what="dit fused chain", mask=np.broadcast_to(keep_c, ref.shape))
