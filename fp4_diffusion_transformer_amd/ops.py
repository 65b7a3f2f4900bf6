"""ctypes binding of libfp4dit.so (include/fp4dit.h).

Argument marshalling only: every step runs in the HIP library.  Tensors must
be contiguous and on the ROCm device; outputs are allocated with torch and
filled by the library on torch's current stream.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

F32 = 0
BF16 = 1
F16 = 2
ROWMAJOR = 0
TILED = 1
_LAYOUTS = {"rowmajor": ROWMAJOR, "tiled": TILED}
_STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "misaligned pointer",
           4: "unsupported argument", 5: "kernel launch failed"}

_lib_handle = None


class Fp4ditError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, _STATUS.get(status, "unknown"), status))
        self.status = status


def library_path():
    return os.path.join(_HERE, "libfp4dit.so")


def lib():
    """The loaded library with typed entry points (loaded on first use)."""
    global _lib_handle
    if _lib_handle is None:
        path = library_path()
        if not os.path.exists(path):
            raise Fp4ditError("load", 4) from FileNotFoundError(
                path + " is not built: run python -m fp4_diffusion_transformer_amd.build")
        L = ctypes.CDLL(path)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        sig = {
            "fp4dit_quantize_mxfp4": [P, I32, I64, I64, P, P, I32, P],
            "fp4dit_block_transform": [P, I32, I64, I64, P, I64, P, I32, P, P, I32, P],
            "fp4dit_fold_inverse_transform": [P, I64, I64, P, I64, P, P],
            "fp4dit_mx_relayout": [P, P, I32, I64, I64, P, P, I32, P],
            "fp4dit_pack_weight": [P, I32, I64, I64, I32, P, P, I32, P],
            "fp4dit_gemm_fp4_epilogue_none": [I64, I64, I64, P, P, P, P, P, I32, P],
            "fp4dit_gemm_fp4_epilogue_rmsnorm_head": [I64, I64, I64, P, P, P, P, I32, I64, P, F, P, I32, P],
            "fp4dit_gemm_fp4_epilogue_swiglu": [I64, I64, I64, P, P, P, P, P, I32, P, P, P],
            "fp4dit_gemm_fp4_epilogue_swiglu_transform": [I64, I64, I64, P, P, P, P, P, I64, P, I32, P, P, P],
            "fp4dit_rmsnorm_head": [P, I64, I64, I32, I64, P, F, P, P],
            "fp4dit_swiglu": [P, I64, I64, I32, P, P],
            "fp4dit_fake_quantize_mxfp4": [P, I32, I64, I64, P, I32, P],
            "fp4dit_etd1_update": [P, P, I64, I32, F, F, P, P],
            "fp4dit_etd2_update": [P, P, P, I64, I32, F, F, F, P, P],
            "fp4dit_richardson_combine": [P, P, I64, I32, F, P, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        D, PD = ctypes.c_double, ctypes.POINTER(ctypes.c_double)
        L.fp4dit_etd_coefficients.argtypes = [D, D, D, D, I32, I32, PD, PD, PD]
        L.fp4dit_etd_coefficients.restype = ctypes.c_int
        L.fp4dit_swiglu_interleave_group.argtypes = []
        L.fp4dit_swiglu_interleave_group.restype = ctypes.c_int32
        L.fp4dit_status_string.argtypes = [ctypes.c_int]
        L.fp4dit_status_string.restype = ctypes.c_char_p
        _lib_handle = L
    return _lib_handle


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise Fp4ditError(name, st)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(name + " must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(name + " must be contiguous")
    return t


def _dtype_code(dt, allow_f16=False):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    if allow_f16 and dt == torch.float16:
        return F16
    raise ValueError("dtype must be float32 or bfloat16%s, got %s" % (" or float16" if allow_f16 else "", dt))


def swiglu_interleave_group():
    return int(lib().fp4dit_swiglu_interleave_group())


class MxTensor(NamedTuple):
    """An MXFP4 matrix [rows, cols]: codes and e8m0 scales in `layout`.

    For "tiled" the buffers are padded (codes to an even number of rows,
    scales to a multiple of 32 rows), so rows/cols are the logical shape.
    """
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int
    layout: str = "tiled"


def _round_up(v, m):
    return (v + m - 1) // m * m


def mx_empty(rows, cols, layout="tiled", device="cuda"):
    """Allocate an MxTensor of the right storage size for `layout`."""
    if layout == "tiled":
        codes = torch.empty((_round_up(rows, 2), cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((_round_up(rows, 32), cols // 32), dtype=torch.uint8, device=device)
    elif layout == "rowmajor":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
    else:
        raise ValueError("layout must be 'tiled' or 'rowmajor'")
    return MxTensor(codes, scales, rows, cols, layout)


def _mx_bytes(rows, cols, layout):
    if layout == "tiled":
        return _round_up(rows, 2) * (cols // 2), _round_up(rows, 32) * (cols // 32)
    return rows * (cols // 2), rows * (cols // 32)


def _mx_check(mx: MxTensor, rows, cols, name):
    """An MxTensor the library will read or write as [rows, cols]: uint8,
    contiguous device buffers at least as large as its layout needs (the
    C ABI takes bare pointers and cannot check sizes)."""
    if mx.layout not in _LAYOUTS:
        raise ValueError(name + ".layout must be 'tiled' or 'rowmajor'")
    if mx.rows != rows or mx.cols != cols:
        raise ValueError("%s is [%d, %d], expected [%d, %d]" % (name, mx.rows, mx.cols, rows, cols))
    need = _mx_bytes(rows, cols, mx.layout)
    for t, nm, n in ((mx.codes, name + ".codes", need[0]), (mx.scales, name + ".scales", need[1])):
        _dev(t, nm)
        if t.dtype != torch.uint8:
            raise ValueError(nm + " must be uint8")
        if t.numel() < n:
            raise ValueError("%s holds %d bytes, needs %d" % (nm, t.numel(), n))
    return mx


def _out_check(t, shape, dtypes, name):
    """A caller-given output tensor: on the device, contiguous, of `shape`
    and one of `dtypes`."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s must be one of %s, got %s" % (name, dtypes, t.dtype))
    return t


_F32_BF16 = (torch.float32, torch.bfloat16)


def quantize_mxfp4(x, layout="tiled", out: Optional[MxTensor] = None):
    """x [rows, cols] float32/bfloat16 -> MxTensor."""
    _dev(x, "x")
    rows, cols = x.shape
    mx = _mx_check(out, rows, cols, "out") if out is not None else mx_empty(rows, cols, layout, x.device)
    _call("fp4dit_quantize_mxfp4", _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(mx.codes), _ptr(mx.scales),
          _LAYOUTS[mx.layout], _stream())
    return mx


def block_transform(x, t, y_dtype=None, quantize=True, layout="tiled", y=None, out: Optional[MxTensor] = None):
    """y_b = x_b @ T_b per 32-element block.  t: bfloat16 [n_t, 32, 32].

    Returns (y or None, MxTensor or None): y is produced when y_dtype
    (float32 / bfloat16) or a y tensor is given, the MXFP4 encoding of the
    product when quantize is set (into `out` if given).
    """
    _dev(x, "x")
    _dev(t, "t")
    if t.dtype != torch.bfloat16:
        raise ValueError("t must be bfloat16")
    rows, cols = x.shape
    if y is None and y_dtype is not None:
        y = torch.empty((rows, cols), dtype=y_dtype, device=x.device)
    elif y is not None:
        _out_check(y, (rows, cols), _F32_BF16, "y")
    mx = None
    if quantize:
        mx = _mx_check(out, rows, cols, "out") if out is not None else mx_empty(rows, cols, layout, x.device)
    _call("fp4dit_block_transform", _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(t), t.shape[0],
          _ptr(y), _dtype_code(y.dtype) if y is not None else F32,
          _ptr(mx.codes) if mx else None, _ptr(mx.scales) if mx else None,
          _LAYOUTS[mx.layout] if mx else TILED, _stream())
    return y, mx


def mx_relayout(mx: MxTensor, layout="tiled", out: Optional[MxTensor] = None):
    """The same MXFP4 values in another byte layout ("tiled": the GEMM's
    operand layout; "rowmajor": plain codes [rows, cols/2], scales
    [rows, cols/32])."""
    _mx_check(mx, mx.rows, mx.cols, "mx")
    res = _mx_check(out, mx.rows, mx.cols, "out") if out is not None else \
        mx_empty(mx.rows, mx.cols, layout, mx.codes.device)
    _call("fp4dit_mx_relayout", _ptr(mx.codes), _ptr(mx.scales), _LAYOUTS[mx.layout], mx.rows, mx.cols,
          _ptr(res.codes), _ptr(res.scales), _LAYOUTS[res.layout], _stream())
    return res


def fold_inverse_transform(w, t):
    """W'_b = T_b^-1 @ W_b for the 32-row blocks of w [K, N] float32."""
    _dev(w, "w")
    _dev(t, "t")
    if w.dtype != torch.float32 or t.dtype != torch.bfloat16:
        raise ValueError("w must be float32 and t bfloat16")
    k, n = w.shape
    out = torch.empty_like(w)
    _call("fp4dit_fold_inverse_transform", _ptr(w), k, n, _ptr(t), t.shape[0], _ptr(out), _stream())
    return out


def pack_weight(w, interleave_group=0, layout="tiled"):
    """Logical weight w [K, N] -> MXFP4 [N, K] (rows = physical output columns).

    interleave_group > 0 treats w as [gate | up] and interleaves the columns
    for the SwiGLU epilogue (use swiglu_interleave_group()).
    """
    _dev(w, "w")
    k, n = w.shape
    mx = mx_empty(n, k, layout, w.device)
    _call("fp4dit_pack_weight", _ptr(w), _dtype_code(w.dtype), k, n, int(interleave_group), _ptr(mx.codes),
          _ptr(mx.scales), _LAYOUTS[layout], _stream())
    return mx


def _gemm_shapes(a: MxTensor, b: MxTensor):
    for t, nm in ((a.codes, "a.codes"), (a.scales, "a.scales"), (b.codes, "b.codes"), (b.scales, "b.scales")):
        _dev(t, nm)
        if t.dtype != torch.uint8:
            raise ValueError(nm + " must be uint8")
    if a.layout != "tiled" or b.layout != "tiled":
        raise ValueError("GEMM operands must be in the tiled layout")
    if a.cols != b.cols:
        raise ValueError("A and B disagree on K")
    _mx_check(a, a.rows, a.cols, "a")
    _mx_check(b, b.rows, b.cols, "b")
    return a.rows, b.rows, a.cols


def gemm_fp4_epilogue_none(a: MxTensor, b: MxTensor, out_dtype=torch.bfloat16, out=None):
    m, n, k = _gemm_shapes(a, b)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.codes.device)
    _out_check(out, (m, n), _F32_BF16, "out")
    _call("fp4dit_gemm_fp4_epilogue_none", m, n, k, _ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales),
          _ptr(out), _dtype_code(out.dtype), _stream())
    return out


def gemm_fp4_epilogue_rmsnorm_head(a: MxTensor, b: MxTensor, head_dim, n_norm_cols, norm_w, eps=1e-6,
                                   out_dtype=torch.bfloat16, out=None):
    m, n, k = _gemm_shapes(a, b)
    if norm_w is not None:
        _dev(norm_w, "norm_w")
        if norm_w.dtype != torch.float32:
            raise ValueError("norm_w must be float32")
    if norm_w is not None and norm_w.numel() < int(n_norm_cols):
        raise ValueError("norm_w holds %d gains, needs %d" % (norm_w.numel(), int(n_norm_cols)))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.codes.device)
    _out_check(out, (m, n), _F32_BF16, "out")
    _call("fp4dit_gemm_fp4_epilogue_rmsnorm_head", m, n, k, _ptr(a.codes), _ptr(a.scales), _ptr(b.codes),
          _ptr(b.scales), int(head_dim), int(n_norm_cols), _ptr(norm_w), float(eps), _ptr(out),
          _dtype_code(out.dtype), _stream())
    return out


def gemm_fp4_epilogue_swiglu(a: MxTensor, b: MxTensor, out_dtype=torch.bfloat16, requant=False, out=None,
                             out_mx: Optional[MxTensor] = None):
    """SwiGLU over an interleaved weight.  Returns (h or None, MxTensor or None):
    h [M, N/2] when out_dtype (or `out`) is given, its tiled MXFP4 encoding
    when requant is set (into `out_mx` if given)."""
    m, n, k = _gemm_shapes(a, b)
    h = out
    if h is None and out_dtype is not None:
        h = torch.empty((m, n // 2), dtype=out_dtype, device=a.codes.device)
    elif h is not None:
        _out_check(h, (m, n // 2), _F32_BF16, "out")
    mx = None
    if requant:
        mx = out_mx if out_mx is not None else mx_empty(m, n // 2, "tiled", a.codes.device)
        if mx.layout != "tiled":
            raise ValueError("the requantised output is tiled")
        _mx_check(mx, m, n // 2, "out_mx")
    _call("fp4dit_gemm_fp4_epilogue_swiglu", m, n, k, _ptr(a.codes), _ptr(a.scales), _ptr(b.codes),
          _ptr(b.scales), _ptr(h), _dtype_code(h.dtype) if h is not None else F32,
          _ptr(mx.codes) if mx else None, _ptr(mx.scales) if mx else None, _stream())
    return h, mx


def gemm_fp4_epilogue_swiglu_transform(a: MxTensor, b: MxTensor, t, y_dtype=None, y=None,
                                       out_mx: Optional[MxTensor] = None):
    """SwiGLU over an interleaved weight, block-transformed by t (bfloat16
    [n_t, 32, 32], y_b = h_b @ T_b) and quantised.  Returns (y or None,
    MxTensor): y [M, N/2] when y_dtype (or `y`) is given, and the tiled MXFP4
    encoding of y (into `out_mx` if given)."""
    m, n, k = _gemm_shapes(a, b)
    _dev(t, "t")
    if t.dtype != torch.bfloat16:
        raise ValueError("t must be bfloat16")
    if y is None and y_dtype is not None:
        y = torch.empty((m, n // 2), dtype=y_dtype, device=a.codes.device)
    elif y is not None:
        _out_check(y, (m, n // 2), _F32_BF16, "y")
    mx = out_mx if out_mx is not None else mx_empty(m, n // 2, "tiled", a.codes.device)
    if mx.layout != "tiled":
        raise ValueError("the requantised output is tiled")
    _mx_check(mx, m, n // 2, "out_mx")
    _call("fp4dit_gemm_fp4_epilogue_swiglu_transform", m, n, k, _ptr(a.codes), _ptr(a.scales), _ptr(b.codes),
          _ptr(b.scales), _ptr(t), t.shape[0], _ptr(y), _dtype_code(y.dtype) if y is not None else F32,
          _ptr(mx.codes), _ptr(mx.scales), _stream())
    return y, mx


def rmsnorm_head(x, head_dim, n_norm_cols, norm_w, eps=1e-6, out=None):
    """Unfused per-head RMSNorm of a bf16 [rows, cols] tensor (bf16 result)."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    if norm_w is not None:
        _dev(norm_w, "norm_w")
        if norm_w.dtype != torch.float32:
            raise ValueError("norm_w must be float32")
    rows, cols = x.shape
    if norm_w is not None and norm_w.numel() < int(n_norm_cols):
        raise ValueError("norm_w holds %d gains, needs %d" % (norm_w.numel(), int(n_norm_cols)))
    if out is None:
        out = torch.empty_like(x)
    _out_check(out, (rows, cols), (torch.bfloat16,), "out")
    _call("fp4dit_rmsnorm_head", _ptr(x), rows, cols, int(head_dim), int(n_norm_cols), _ptr(norm_w), float(eps),
          _ptr(out), _stream())
    return out


def swiglu(c, group, out=None):
    """Unfused SwiGLU of a bf16 [rows, n_phys] interleaved GEMM output -> bf16 [rows, n_phys/2]."""
    _dev(c, "c")
    if c.dtype != torch.bfloat16:
        raise ValueError("c must be bfloat16")
    rows, n_phys = c.shape
    if out is None:
        out = torch.empty((rows, n_phys // 2), dtype=torch.bfloat16, device=c.device)
    _out_check(out, (rows, n_phys // 2), (torch.bfloat16,), "out")
    _call("fp4dit_swiglu", _ptr(c), rows, n_phys, int(group), _ptr(out), _stream())
    return out


# ------------------------------------------------------------------- QAD --
def fake_quantize_mxfp4(x, y_dtype=None, out=None):
    """y = D(Q(x)) per 32-element block of each row (float32 / bfloat16)."""
    _dev(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=y_dtype or x.dtype, device=x.device)
    _out_check(out, (rows, cols), _F32_BF16, "out")
    _call("fp4dit_fake_quantize_mxfp4", _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(out),
          _dtype_code(out.dtype), _stream())
    return out


class _FakeQuantSTE(torch.autograd.Function):
    """Forward: the fake-quantisation kernel.  Backward: the straight-through
    estimator hands the incoming gradient on unchanged."""

    @staticmethod
    def forward(ctx, x):
        return fake_quantize_mxfp4(x.contiguous())

    @staticmethod
    def backward(ctx, grad_y):
        return grad_y


def fake_quantize_ste(x):
    return _FakeQuantSTE.apply(x)


# --------------------------------------------------------------- sampler --
def _same(ts, names):
    for t, nm in zip(ts, names):
        _dev(t, nm)
        if t.dtype != ts[0].dtype or t.numel() != ts[0].numel():
            raise ValueError("%s must match %s in dtype and size" % (nm, names[0]))
    return _dtype_code(ts[0].dtype, allow_f16=True), ts[0].numel()


def etd1_update(x, x0, decay, coeff, out=None):
    """out = decay * x + coeff * x0 (elementwise, fp32 arithmetic)."""
    code, n = _same([x, x0], ["x", "x0"])
    if out is None:
        out = torch.empty_like(x)
    _same([x, out], ["x", "out"])
    _call("fp4dit_etd1_update", _ptr(x), _ptr(x0), n, code, float(decay), float(coeff), _ptr(out), _stream())
    return out


def etd2_update(x, x0, x0_prev, decay, c0, c1, out=None):
    """out = decay * x + c0 * x0 + c1 * x0_prev."""
    code, n = _same([x, x0, x0_prev], ["x", "x0", "x0_prev"])
    if out is None:
        out = torch.empty_like(x)
    _same([x, out], ["x", "out"])
    _call("fp4dit_etd2_update", _ptr(x), _ptr(x0), _ptr(x0_prev), n, code, float(decay), float(c0), float(c1),
          _ptr(out), _stream())
    return out


def richardson_combine(fine, coarse, scale, out=None):
    """out = (scale * fine - coarse) / (scale - 1); scale = 2^p."""
    code, n = _same([fine, coarse], ["fine", "coarse"])
    if out is None:
        out = torch.empty_like(fine)
    _same([fine, out], ["fine", "out"])
    _call("fp4dit_richardson_combine", _ptr(fine), _ptr(coarse), n, code, float(scale), _ptr(out), _stream())
    return out


def etd_coefficients(alpha_s, sigma_s, alpha_t, sigma_t, order=1, first_step=False):
    """(decay, c0, c1) of one ETD step (host arithmetic in the library)."""
    d, c0, c1 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _call("fp4dit_etd_coefficients", float(alpha_s), float(sigma_s), float(alpha_t), float(sigma_t), int(order),
          int(bool(first_step)), ctypes.byref(d), ctypes.byref(c0), ctypes.byref(c1))
    return d.value, c0.value, c1.value
