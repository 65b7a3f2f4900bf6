"""MI355X (gfx950) fused MXFP4 GEMM + epilogue for diffusion-transformer linears.

The compute lives in the HIP library libfp4dit.so behind a C ABI
(include/fp4dit.h); `ops` is a thin ctypes binding over it that takes torch
tensors for device memory and streams.  The library is loaded on first use
and its absence raises: there is no CPU fallback.
"""

from .ops import (  # noqa: F401
    Fp4ditError,
    MxTensor,
    mx_empty,
    block_transform,
    fold_inverse_transform,
    gemm_fp4_epilogue_none,
    gemm_fp4_epilogue_rmsnorm_head,
    gemm_fp4_epilogue_swiglu,
    lib,
    library_path,
    pack_weight,
    quantize_mxfp4,
    swiglu_interleave_group,
)
