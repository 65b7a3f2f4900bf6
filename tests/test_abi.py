"""The C-ABI library loads, exports what include/fp4dit.h declares, and
rejects bad arguments on the host (no GPU needed: nothing is launched).

Every call below carries at least one invalid argument, so validation
returns before any HIP call; the fake addresses are never dereferenced."""

import ctypes
import os
import re

import pytest

from fp4_diffusion_transformer_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4dit.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_UNSUP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ROWMAJOR, TILED = 0, 1
P = 0x10000          # a fake, 64 KiB-aligned "device" address: never dereferenced
P_ODD = 0x10001


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4dit_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.library_path()):
        pytest.fail("libfp4dit.so is not built (python -m fp4_diffusion_transformer_amd.build)")
    return ops.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 18
    assert "fp4dit_mx_relayout" in names and "fp4dit_clock_probe" not in names
    raw = ctypes.CDLL(ops.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings_and_group(L):
    assert L.fp4dit_status_string(0) == b"ok"
    assert L.fp4dit_status_string(2) == b"invalid shape"
    assert L.fp4dit_swiglu_interleave_group() == 32


def test_quantize_validation(L):
    q = L.fp4dit_quantize_mxfp4
    assert q(P, F32, 4, 48, P, P, ROWMAJOR, None) == E_SHAPE           # cols % 32
    assert q(P, F32, 4, 96, P, P, TILED, None) == E_SHAPE              # tiled: cols % 128
    assert q(P, F32, -1, 64, P, P, ROWMAJOR, None) == E_SHAPE
    assert q(P, 7, 4, 64, P, P, ROWMAJOR, None) == E_UNSUP             # dtype
    assert q(P, F32, 4, 128, P, P, 5, None) == E_UNSUP                 # layout
    assert q(None, BF16, 4, 64, P, P, ROWMAJOR, None) == E_NULL
    assert q(P, BF16, 4, 64, None, P, ROWMAJOR, None) == E_NULL
    assert q(P_ODD, BF16, 4, 64, P, P, ROWMAJOR, None) == E_ALIGN
    assert q(P, BF16, 4, 64, P_ODD, P, ROWMAJOR, None) == E_ALIGN
    assert q(None, BF16, 0, 64, None, None, ROWMAJOR, None) == OK       # empty: nothing to do


def test_gemm_validation(L):
    g = L.fp4dit_gemm_fp4_epilogue_none
    assert g(256, 500, 512, P, P, P, P, P, BF16, None) == E_SHAPE         # N % 256
    assert g(256, 512, 320, P, P, P, P, P, BF16, None) == E_SHAPE         # K % 128
    assert g(256, 512, 128, P, P, P, P, P, BF16, None) == E_SHAPE         # K >= 256
    assert g(256, 512, 0, P, P, P, P, P, BF16, None) == E_SHAPE
    assert g(-1, 512, 512, P, P, P, P, P, BF16, None) == E_SHAPE
    assert g(256, 512, 512, None, P, P, P, P, BF16, None) == E_NULL
    assert g(256, 512, 512, P, P, P, P, None, BF16, None) == E_NULL
    assert g(256, 512, 512, P_ODD, P, P, P, P, BF16, None) == E_ALIGN
    assert g(256, 512, 512, P, P + 2, P, P, P, BF16, None) == E_ALIGN      # scales need 4 bytes
    assert g(256, 512, 512, P, P, P, P, P, 9, None) == E_UNSUP
    assert g(0, 512, 512, None, None, None, None, None, BF16, None) == OK
    assert g(1 << 20, 512, 8192, P, P, P, P, P, BF16, None) == E_SHAPE     # 32-bit operand offsets


def test_rmsnorm_validation(L):
    r = L.fp4dit_gemm_fp4_epilogue_rmsnorm_head
    args = (256, 512, 512, P, P, P, P)
    assert r(*args, 64, 512, P, 1e-6, P, BF16, None) == E_UNSUP            # head_dim
    assert r(*args, 256, 384, P, 1e-6, P, BF16, None) == E_SHAPE           # n_norm % head_dim
    assert r(*args, 128, 640, P, 1e-6, P, BF16, None) == E_SHAPE           # n_norm > N
    assert r(*args, 128, 512, None, 1e-6, P, BF16, None) == E_NULL
    assert r(*args, 128, 512, P + 4, 1e-6, P, BF16, None) == E_ALIGN
    assert r(*args, 128, 512, P, -1.0, P, BF16, None) == E_UNSUP           # eps < 0
    assert r(*args, 128, 512, P, float("nan"), P, BF16, None) == E_UNSUP


def test_swiglu_validation(L):
    s = L.fp4dit_gemm_fp4_epilogue_swiglu
    args = (256, 512, 512, P, P, P, P)
    assert s(*args, None, BF16, None, None, None) == E_NULL                # no output at all
    assert s(*args, None, BF16, P, None, None) == E_UNSUP                  # codes without scales
    assert s(*args, P_ODD, BF16, None, None, None) == E_ALIGN


def test_swiglu_transform_validation(L):
    s = L.fp4dit_gemm_fp4_epilogue_swiglu_transform
    args = (256, 512, 512, P, P, P, P)
    assert s(*args, P, 3, None, F32, P, P, None) == E_SHAPE                # n_t not 1 or N/64
    assert s(*args, None, 8, None, F32, P, P, None) == E_NULL              # no T (n_t = N/64)
    assert s(*args, P, 1, None, F32, None, P, None) == E_NULL              # codes are required
    assert s(*args, P, 1, None, F32, P, None, None) == E_NULL
    assert s(*args, P_ODD, 1, None, F32, P, P, None) == E_ALIGN            # T is bf16
    assert s(*args, P, 1, P_ODD, BF16, P, P, None) == E_ALIGN
    assert s(*args, P, 1, None, F32, P, P_ODD, None) == E_ALIGN            # scales pair: 2 bytes
    assert s(*args, P, 1, P, 9, P, P, None) == E_UNSUP
    assert s(256, 320, 512, P, P, P, P, P, 1, None, F32, P, P, None) == E_SHAPE   # N % 256
    assert s(0, 512, 512, None, None, None, None, None, 1, None, F32, None, None, None) == OK


def test_unfused_validation(L):
    r = L.fp4dit_rmsnorm_head
    assert r(P, 4, 512, 64, 512, P, 1e-6, P, None) == E_UNSUP                # head_dim
    assert r(P, 4, 384, 256, 256, P, 1e-6, P, None) == E_SHAPE               # cols % head_dim
    assert r(P, 4, 512, 128, 640, P, 1e-6, P, None) == E_SHAPE               # n_norm > cols
    assert r(P, 4, 512, 128, 384, None, 1e-6, P, None) == E_NULL
    assert r(P, 4, 512, 128, 0, None, 1e-6, None, None) == E_NULL            # no output
    assert r(P + 8, 4, 512, 128, 384, P, 1e-6, P, None) == E_ALIGN
    assert r(P, 4, 512, 128, 384, P, float("inf"), P, None) == E_UNSUP
    assert r(None, 0, 512, 128, 384, None, 1e-6, None, None) == OK           # empty
    sw = L.fp4dit_swiglu
    assert sw(P, 4, 512, 12, P + 4096, None) == E_UNSUP                       # group % 8
    assert sw(P, 4, 96, 32, P + 4096, None) == E_SHAPE                        # n_phys % 2g
    assert sw(P, 4, 512, 32, P + 1024, None) == E_UNSUP                       # h overlaps c
    assert sw(P, 4, 512, 32, P + 4104, None) == E_ALIGN
    assert sw(None, 4, 512, 32, P, None) == E_NULL
    assert sw(None, 0, 512, 32, None, None) == OK


def test_fake_quant_validation(L):
    f = L.fp4dit_fake_quantize_mxfp4
    assert f(P, BF16, 4, 48, P + 4096, BF16, None) == E_SHAPE                 # cols % 32
    assert f(P, 2, 4, 64, P + 4096, BF16, None) == E_UNSUP                    # F16 is for the sampler only
    assert f(P, BF16, 4, 64, P, F32, None) == E_UNSUP                         # in place across dtypes
    assert f(P, F32, 4, 64, P + 512, BF16, None) == E_UNSUP                   # overlap (x spans 1 KiB)
    assert f(P, BF16, 4, 64, P + 4104, BF16, None) == E_ALIGN
    assert f(None, BF16, 4, 64, P, BF16, None) == E_NULL
    assert f(None, BF16, 0, 64, None, BF16, None) == OK


def test_sampler_validation(L):
    F16 = 2
    e1, e2, rc = L.fp4dit_etd1_update, L.fp4dit_etd2_update, L.fp4dit_richardson_combine
    assert e1(P, P + 4096, 100, 7, 0.5, 0.5, P + 8192, None) == E_UNSUP       # dtype
    assert e1(P, P + 4096, -1, F16, 0.5, 0.5, P + 8192, None) == E_SHAPE
    assert e1(P, None, 100, F16, 0.5, 0.5, P + 8192, None) == E_NULL
    assert e1(P, P + 4096, 100, F32, 0.5, 0.5, P + 200, None) == E_UNSUP     # out overlaps x
    # out == x passes the overlap check (the misaligned x0 is what fails)
    assert e1(P, P + 4100, 100, F32, 0.5, 0.5, P, None) == E_ALIGN
    assert e1(P + 4, P + 4096, 100, F32, 0.5, 0.5, P + 8192, None) == E_ALIGN
    assert e2(P, P + 4096, None, 100, BF16, 0.5, 0.3, 0.1, P + 8192, None) == E_NULL
    assert rc(P, P + 4096, 100, F32, 1.0, P + 8192, None) == E_UNSUP          # scale 1
    assert rc(None, None, 0, F32, 2.0, None, None) == OK


def test_sizes_too_large_for_int64_products(L):
    """Sizes whose products would overflow int64 are rejected before any
    arithmetic on them (each size must be below 2^31)."""
    big = 1 << 40
    assert L.fp4dit_quantize_mxfp4(P, BF16, big, big, P, P, ROWMAJOR, None) == E_SHAPE
    assert L.fp4dit_fake_quantize_mxfp4(P, BF16, big, big, P, BF16, None) == E_SHAPE
    assert L.fp4dit_rmsnorm_head(P, big, 128 * big, 128, 0, None, 1e-6, P, None) == E_SHAPE
    assert L.fp4dit_swiglu(P, big, 64 * big, 32, P, None) == E_SHAPE
    assert L.fp4dit_gemm_fp4_epilogue_none(big, 256, 256, P, P, P, P, P, BF16, None) == E_SHAPE
    assert L.fp4dit_pack_weight(P, F32, 128 * big, big, 0, P, P, TILED, None) == E_SHAPE
    assert L.fp4dit_block_transform(P, BF16, big, 128 * big, P, 1, None, BF16, P, P, TILED, None) == E_SHAPE
    assert L.fp4dit_fold_inverse_transform(P, 32 * big, big, P, 1, P + 64, None) == E_SHAPE


def test_clock_probe_validation():
    """The measurement helper lives in its own library, not in libfp4dit.so."""
    from fp4_diffusion_transformer_amd import clockprobe
    assert not hasattr(ctypes.CDLL(ops.library_path()), "fp4dit_clock_probe")
    c = clockprobe.lib().fp4dit_clock_probe
    assert c(None, 1, 100, None) == E_NULL
    assert c(P + 4, 1, 100, None) == E_ALIGN
    assert c(P, 0, 100, None) == E_SHAPE
    assert c(P, 65537, 100, None) == E_SHAPE
    assert c(P, 1, 0, None) == E_SHAPE
    assert c(P, 1, (1 << 20) + 1, None) == E_SHAPE


def test_etd_coefficients_host_logic(L):
    """The host helper against the oracle's coefficients (no GPU involved)."""
    import math
    from oracle import sampler

    def vp(t):
        a = math.cos(0.5 * math.pi * t)
        return a, math.sqrt(1.0 - a * a)

    d, c0, c1 = (ctypes.c_double() for _ in range(3))
    for s, t in [(0.9, 0.8), (0.5, 0.3), (0.2, 0.05)]:
        args = (*vp(s), *vp(t))
        for order, first in [(1, 0), (2, 1), (2, 0)]:
            assert L.fp4dit_etd_coefficients(*args, order, first, ctypes.byref(d), ctypes.byref(c0),
                                             ctypes.byref(c1)) == OK
            if order == 1:
                ref = sampler.etd1_coefficients(*args) + (0.0,)
            else:
                ref = sampler.etd2_coefficients(*args, first_step=bool(first))
            assert (d.value, c0.value, c1.value) == pytest.approx(ref, rel=1e-14, abs=1e-300)
    assert L.fp4dit_etd_coefficients(0.5, 0.5, 0.6, 0.4, 3, 0, ctypes.byref(d), ctypes.byref(c0),
                                     ctypes.byref(c1)) == E_UNSUP
    assert L.fp4dit_etd_coefficients(0.5, 0.0, 0.6, 0.4, 1, 0, ctypes.byref(d), ctypes.byref(c0),
                                     ctypes.byref(c1)) == E_SHAPE
    assert L.fp4dit_etd_coefficients(0.5, 0.5, 0.6, 0.4, 1, 0, None, ctypes.byref(c0), ctypes.byref(c1)) == E_NULL


def test_relayout_validation(L):
    r = L.fp4dit_mx_relayout
    Q = P + (1 << 20)                                   # a second fake buffer, far from P
    assert r(P, P + 4096, ROWMAJOR, 4, 96, Q, Q + 4096, TILED, None) == E_SHAPE     # tiled side: cols % 128
    assert r(P, P + 4096, ROWMAJOR, 4, 80, Q, Q + 4096, ROWMAJOR, None) == E_SHAPE  # cols % 32
    assert r(P, P + 4096, ROWMAJOR, -1, 128, Q, Q + 4096, TILED, None) == E_SHAPE
    assert r(P, P + 4096, 3, 4, 128, Q, Q + 4096, TILED, None) == E_UNSUP
    assert r(P, P + 4096, ROWMAJOR, 4, 128, Q, Q + 4096, 7, None) == E_UNSUP
    assert r(None, P + 4096, ROWMAJOR, 4, 128, Q, Q + 4096, TILED, None) == E_NULL
    assert r(P, P + 4096, ROWMAJOR, 4, 128, Q, None, TILED, None) == E_NULL
    assert r(P_ODD, P + 4096, ROWMAJOR, 4, 128, Q, Q + 4096, TILED, None) == E_ALIGN
    assert r(P, P + 4096, ROWMAJOR, 4, 128, Q + 8, Q + 4096, TILED, None) == E_ALIGN
    assert r(P, P + 4096, ROWMAJOR, 4, 128, P, Q + 4096, TILED, None) == E_UNSUP    # output is the input
    assert r(P, P + 4096, ROWMAJOR, 4, 128, P + 128, Q, TILED, None) == E_UNSUP     # overlaps the input
    assert r(P, P + 4096, ROWMAJOR, 4, 128, Q, Q + 16, TILED, None) == E_UNSUP      # outputs overlap
    assert r(None, None, ROWMAJOR, 0, 128, None, None, TILED, None) == OK          # empty


def test_transform_pack_fold_validation(L):
    bt = L.fp4dit_block_transform
    assert bt(P, BF16, 8, 96, P, 2, P, F32, None, None, TILED, None) == E_SHAPE   # n_t not 1 or cols/32
    assert bt(P, BF16, 8, 96, P, 3, None, F32, None, None, TILED, None) == E_NULL  # no output
    assert bt(P, BF16, 8, 96, P, 1, None, F32, P, None, TILED, None) == E_UNSUP   # codes without scales
    assert bt(P, BF16, 8, 80, P, 1, P, F32, None, None, TILED, None) == E_SHAPE
    assert bt(P, BF16, 8, 96, P, 1, None, F32, P, P, TILED, None) == E_SHAPE      # tiled: cols % 128
    pw = L.fp4dit_pack_weight
    assert pw(P, F32, 64, 96, 32, P, P, ROWMAJOR, None) == E_SHAPE                # N % 2g
    assert pw(P, F32, 48, 64, 0, P, P, ROWMAJOR, None) == E_SHAPE                 # K % 32
    assert pw(P, F32, 64, 64, 0, P, P, TILED, None) == E_SHAPE                    # tiled: K % 128
    assert pw(P, F32, 64, 64, -1, P, P, ROWMAJOR, None) == E_UNSUP
    fo = L.fp4dit_fold_inverse_transform
    assert fo(P, 64, 16, P, 3, P + 64, None) == E_SHAPE
    assert fo(P, 64, 16, P, 2, P, None) == E_UNSUP                          # aliasing
    assert fo(None, 64, 16, P, 2, P + 64, None) == E_NULL
