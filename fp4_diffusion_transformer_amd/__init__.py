"""MI355X (gfx950) fused MXFP4 GEMM + epilogue for diffusion-transformer linears."""
