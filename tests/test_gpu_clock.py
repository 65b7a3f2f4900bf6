"""The shader-clock probe (libfp4dit_clock.so, built apart from the method's
library), a measurement helper that bench.py uses to quote
the MXFP4 roofline at the clock the box sustains under an FP4 MFMA load:
both counters advance at plausible rates, and the whole-chip load runs no
faster than one lightly loaded workgroup."""

import numpy as np
import pytest
import torch

from gpu_util import announce
from fp4_diffusion_transformer_amd import clockprobe

pytestmark = pytest.mark.gpu


def test_clock_probe_counts_and_clocks():
    announce("clock probe")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(12 * cus, dtype=torch.int64, device="cuda")
    clockprobe.clock_probe(out, cus, 256)
    torch.cuda.synchronize()
    v = out.cpu().reshape(-1, 3).numpy()
    assert (v[:, 0] > 256 * 16).all() and (v[:, 1] > 0).all()   # at least a tick per MFMA
    loaded = float(np.median(clockprobe.clock_ghz(out, cus)))
    light = clockprobe.shader_clock_ghz(1, 64)
    assert 0.3 < loaded < 3.0 and 0.3 < light < 3.0, (loaded, light)   # published maximum 2.4 GHz
    assert loaded <= light * 1.05, (loaded, light)
