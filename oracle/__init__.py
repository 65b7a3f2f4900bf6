"""CPU oracle for the fused MXFP4 GEMM + epilogue path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, tables, helpers or pre/post-processing); it depends on
NumPy and the Python standard library only.

Everything here is plain, slow and written to be checked against the pages
by eye: float64 arithmetic, vectorised NumPy where the definition is
elementwise, a library matmul / linear solve where the definition is a plain
product.  Sources:

* fal, "Serving sub-second Ideogram v4 without quality loss" (P1):
  section "Running the transformer in FP4" (the e2m1 bit split), the
  epilogue-fusion sections (RMSNorm formula, per-head reduction, head_dim 256
  revisit schedule) and the gated-SiLU section (SwiGLU formula, column
  interleave at weight-packing time).
* sns.style summary of KroQuant (P3): sections "Background and overview"
  (invertible transform on activations, inverse on weights) and "Deep
  analysis" (32-element block-local learned transform, MXFP4 W4A4).
* fal, QAD section: fake quantisation with a straight-through gradient.
* "拡散サンプリングの高速化：数値計算手法とスコアベースモデルの出会い" (P4):
  the ETD1 / ETD2 updates and the Richardson combine.

Modules:
  mxfp4      e2m1 table, e8m0 scales, block quantise / dequantise
  gemm       dequantise-then-fp64 GEMM and the epilogues (none, per-head
             RMSNorm, SwiGLU with column interleave, MXFP4 re-quantisation)
  transform  32-element block-local transform and its weight-side fold
  bf16       round-to-nearest-even float64 -> bfloat16 for output compares
  qad        MXFP4 fake quantisation (forward) and its straight-through
             gradient (backward)
  sampler    ETD1 / ETD2 sampler updates and the Richardson combine

Every function is pinned by a CPU test (tests/test_oracle_*.py) against
something other than itself: the hand-written code table, exact Fraction
brute force, closed forms and invariants.
"""

from . import bf16, gemm, mxfp4, qad, sampler, transform  # noqa: F401
