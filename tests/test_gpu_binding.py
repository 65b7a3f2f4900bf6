"""The Python binding checks what the C ABI cannot (it takes bare pointers):
caller-given output tensors and MXFP4 buffers must have the shape, dtype and
size the call writes or reads, or it raises before anything is enqueued."""

import pytest
import torch

from gpu_util import announce
from fp4_diffusion_transformer_amd import ops

pytestmark = pytest.mark.gpu


def test_outputs_and_mx_buffers_are_checked():
    announce("binding checks")
    x = torch.randn(64, 256, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):                              # MxTensor of another shape
        ops.quantize_mxfp4(x, out=ops.mx_empty(32, 256))
    short = ops.mx_empty(64, 256)
    short = short._replace(codes=short.codes[:10])
    with pytest.raises(ValueError):                              # codes buffer too small
        ops.quantize_mxfp4(x, out=short)
    a = ops.quantize_mxfp4(x)
    b = ops.pack_weight(torch.randn(256, 256, device="cuda"))
    with pytest.raises(ValueError):                              # out of the wrong shape
        ops.gemm_fp4_epilogue_none(a, b, out=torch.empty(64, 128, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError):                              # out of an unsupported dtype
        ops.gemm_fp4_epilogue_none(a, b, out=torch.empty(64, 256, device="cuda", dtype=torch.float16))
    with pytest.raises(ValueError):                              # operand with a wrong logical shape
        ops.gemm_fp4_epilogue_none(a._replace(rows=128), b)
    with pytest.raises(ValueError):                              # too few norm gains
        ops.gemm_fp4_epilogue_rmsnorm_head(a, b, 128, 256, torch.ones(128, device="cuda"))
    with pytest.raises(ValueError):
        ops.fake_quantize_mxfp4(x, out=torch.empty(64, 128, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        ops.swiglu(x, 32, out=torch.empty(64, 256, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        ops.rmsnorm_head(x, 128, 256, torch.ones(256, device="cuda"), out=torch.empty_like(x).float())
    out = ops.gemm_fp4_epilogue_none(a, b)                       # the defaults still work
    torch.cuda.synchronize()
    assert out.shape == (64, 256)
