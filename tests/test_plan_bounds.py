"""Every direct-to-LDS operand load of the fused GEMM stays inside its buffer.

The GEMM's loads add a scalar stage offset that the hardware's range check
does not cover, so an out-of-range stage would read past the caller's
buffer.  tests/plan_check.cpp walks every load of a launch -- full tiles in
both of their K orders, quarter tiles, every wave, lane and stage -- using
the kernel's own plan code (csrc/gemm_plan.hpp, compiled for the host),
against the tiled buffer sizes, and checks that each K order visits every
stage once.  Runs on the CPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (M, N, K): the workloads' GEMMs and the shapes of the GPU tests, with
# ragged M, the shortest K and K with fewer stages than the quarter loop
# keeps in flight
SHAPES = [(256, 512, 512), (4096, 9216, 3072), (4096, 12288, 4096), (4096, 24576, 3072),
          (16384, 9216, 3072), (16384, 24576, 3072), (16384, 3072, 12288),
          (1, 256, 256), (255, 256, 512), (257, 512, 256), (600, 768, 1024), (1000, 20480, 256),
          (1000, 20480, 512), (1000, 24576, 768), (1000, 256 * 80, 384), (64, 256, 384),
          (300, 768, 384), (300, 768, 640), (300, 768, 1152), (1000, 256 * 96, 384)]


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    subprocess.run([HIPCC if os.path.exists(HIPCC) else "hipcc", "-O2", "-std=c++17",
                    "-I" + os.path.join(ROOT, "fp4_diffusion_transformer_amd", "csrc"),
                    os.path.join(ROOT, "tests", "plan_check.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def test_every_load_in_bounds(plan_check):
    args = [str(v) for s in SHAPES for v in s]
    r = subprocess.run([plan_check] + args, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok ") == len(SHAPES)


def test_walk_catches_unclamped_quarter_stages(plan_check):
    """Without the stage clamp the quarter loop's last loads (and, for
    K = 256, its prologue) read past the end of the operand buffers."""
    for shape in [(4096, 9216, 3072), (1000, 20480, 256)]:
        r = subprocess.run([plan_check, "--unclamped"] + [str(v) for v in shape], capture_output=True, text=True)
        assert r.returncode == 1 and "out of range" in r.stdout, (shape, r.stdout)
