"""Build libfp4dit.so in-tree with hipcc for gfx950 (MI355X).

Every HIP source is compiled to an object in parallel, then linked into a
shared library next to this file.  Usage: python -m fp4_diffusion_transformer_amd.build
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp4dit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of every kernel; the host pass warns
# that it does not know the feature, which is harmless.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-Wno-unused-result"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_clock_probe(verbose)
    build_c_consumer(verbose)
    return LIB


CLOCK_SRC = os.path.join(HERE, "clockprobe", "clock_probe.hip")
CLOCK_LIB = os.path.join(HERE, "libfp4dit_clock.so")


def build_clock_probe(verbose=True):
    """The shader-clock probe, a measurement helper, as a library of its own
    (libfp4dit_clock.so) so that libfp4dit.so holds only the method."""
    tmp = CLOCK_LIB + ".tmp"
    cmd = [HIPCC] + [f for f in FLAGS if not f.startswith("-I")] + [
        "-I" + os.path.dirname(CLOCK_SRC), "-shared", CLOCK_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on the clock probe:\n" + r.stderr)
    os.replace(tmp, CLOCK_LIB)
    if verbose:
        print("built", CLOCK_LIB)
    return CLOCK_LIB


C_CONSUMER_SRC = os.path.join(ROOT, "tests", "c_consumer.c")
C_CONSUMER = os.path.join(ROOT, "tests", "c_consumer")


def build_c_consumer(verbose=True):
    """The plain C program of the C-ABI test, linked against the library
    (C99 with gcc: the header is usable from C)."""
    if not os.path.exists(C_CONSUMER_SRC):
        return None
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I/opt/rocm/include", C_CONSUMER_SRC, "-o", C_CONSUMER, "-L" + HERE, "-lfp4dit", "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../fp4_diffusion_transformer_amd", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed on the C consumer:\n" + r.stderr)
    if verbose:
        print("built", C_CONSUMER)
    return C_CONSUMER


if __name__ == "__main__":
    build()
    sys.exit(0)
