"""ctypes binding of libfp4dit_clock.so: the shader-clock probe, a
measurement helper kept out of the method's library (libfp4dit.so).  bench.py
uses it to quote the MXFP4 roofline at the clock the box sustains under an
FP4 MFMA load."""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib_handle = None


def library_path():
    return os.path.join(_HERE, "libfp4dit_clock.so")


def lib():
    global _lib_handle
    if _lib_handle is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(path + " is not built: run python -m fp4_diffusion_transformer_amd.build")
        L = ctypes.CDLL(path)
        L.fp4dit_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.fp4dit_clock_probe.restype = ctypes.c_int32
        _lib_handle = L
    return _lib_handle


def clock_probe(out, workgroups=1, iters=64):
    """Enqueue the probe on the current stream: `workgroups` x 4 waves of FP4
    MFMAs, each wave writing its s_memtime and 100 MHz s_memrealtime ticks
    (and a checksum) to 3 elements of the int64 device tensor `out`."""
    if (out.dtype != torch.int64 or not out.is_cuda or not out.is_contiguous()
            or out.numel() < 12 * int(workgroups)):
        raise ValueError("clock_probe needs a contiguous int64 CUDA tensor of 12 elements per workgroup")
    st = lib().fp4dit_clock_probe(out.data_ptr(), int(workgroups), int(iters),
                                  torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError("fp4dit_clock_probe failed with status %d" % st)


def clock_ghz(out, workgroups=1):
    """Per-wave shader clocks (GHz) of a finished clock_probe."""
    v = out.flatten()[:12 * int(workgroups)].cpu().reshape(-1, 3).tolist()
    return [0.1 * t / r for t, r, _ in v if r > 0]


def shader_clock_ghz(workgroups=1, iters=64):
    """Median shader clock (GHz) over one probe on the current stream."""
    out = torch.zeros(12 * int(workgroups), dtype=torch.int64, device="cuda")
    clock_probe(out, workgroups, iters)
    c = sorted(clock_ghz(out, workgroups))
    return c[len(c) // 2] if c else float("nan")
