"""Several host threads calling the library at once, each on its own HIP
stream: the entry points keep no mutable state beyond an atomic per-device
CU-count cache, so concurrent calls must give the same bytes as one thread
calling them in turn.  ctypes releases the GIL for the duration of each
foreign call, so the host-side validation and launches really overlap."""

import threading

import numpy as np
import pytest
import torch

import layout
from gpu_util import announce, host
from fp4_diffusion_transformer_amd import ops

pytestmark = pytest.mark.gpu

THREADS, CALLS = 4, 6


def _work(seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(300 + 64 * seed, 512, generator=g).to("cuda", torch.bfloat16)     # ragged, per thread
    w = (torch.randn(512, 512, generator=g) / 512 ** 0.5).cuda()
    wu = (torch.randn(512, 1024, generator=g) / 512 ** 0.5).cuda()
    gains = (torch.rand(256, generator=g) + 0.5).cuda()
    return x, w, wu, gains


def _chain(x, w, wu, gains):
    a = ops.quantize_mxfp4(x)
    q = ops.gemm_fp4_epilogue_rmsnorm_head(a, ops.pack_weight(w), 128, 256, gains, 1e-6)
    _, mx = ops.gemm_fp4_epilogue_swiglu(a, ops.pack_weight(wu, ops.swiglu_interleave_group()), out_dtype=None,
                                         requant=True)
    return a.codes, a.scales, q, mx.codes, mx.scales


def test_concurrent_threads_match_serial():
    inputs = [_work(s) for s in range(THREADS)]
    announce("threads: serial reference", THREADS)
    ref = [[t.clone() for t in _chain(*inp)] for inp in inputs]
    torch.cuda.synchronize()

    results, errors = [None] * THREADS, []
    start = threading.Barrier(THREADS)

    def run(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                start.wait()
                outs = None
                for _ in range(CALLS):
                    outs = _chain(*inputs[i])
                stream.synchronize()
                results[i] = [t.clone() for t in outs]
                stream.synchronize()
        except Exception as e:                           # reported below, with the thread
            errors.append((i, repr(e)))

    announce("threads: concurrent", THREADS, CALLS)
    threads = [threading.Thread(target=run, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(THREADS):
        rows = inputs[i][0].shape[0]                     # even: the tiled code buffers have no padding rows
        got, want = results[i], ref[i]
        assert torch.equal(got[0], want[0]), "thread %d: activation codes" % i
        assert torch.equal(got[2], want[2]), "thread %d: RMSNorm output" % i
        assert torch.equal(got[3], want[3]), "thread %d: SwiGLU requant codes" % i
        for k, cols, what in ((1, 512, "activation scales"), (4, 512, "SwiGLU requant scales")):
            # scale buffers are padded to 32 rows; compare the logical rows
            assert np.array_equal(layout.untile_scales(host(got[k]), rows, cols),
                                  layout.untile_scales(host(want[k]), rows, cols)), "thread %d: %s" % (i, what)
