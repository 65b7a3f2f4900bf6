/*
 * fp4dit.h - C ABI of libfp4dit.so: the MXFP4 (e2m1 values, one e8m0 scale
 * per 32 elements) hot path of a diffusion transformer's linear layers on
 * AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every pointer is a DEVICE pointer to memory the caller allocated and
 *   owns.  The library never allocates, frees, copies to the host or
 *   synchronises: each call enqueues its kernels on `stream` (the null stream
 *   is allowed) and returns.  Outputs are valid once the stream reaches them.
 * - All matrices are dense and row-major, with no leading-dimension padding.
 * - MXFP4 tensors are a pair (codes, scales): 4-bit e2m1 codes
 *   (code = sign<<3 | exp<<1 | mant, exponent bias 1: magnitudes 0, 0.5, 1,
 *   1.5, 2, 3, 4, 6) and one e8m0 scale byte 2^(byte - 127) for each run of
 *   32 consecutive elements of a row.  Two byte layouts (fp4dit_layout):
 *
 *   FP4DIT_MX_ROWMAJOR  codes  uint8 [rows][cols/2], element 2j of a row in
 *                              the low nibble of byte j;
 *                       scales uint8 [rows][cols/32].
 *   FP4DIT_MX_TILED     the layout the GEMM reads (cols % 128 == 0):
 *                       codes in 128-byte tiles of 2 rows x 128 elements;
 *                       tile (r/2, k/128) at byte ((r/2)*(cols/128) + k/128)*128,
 *                       inside it row r%2 at +64*(r%2) and elements k%128
 *                       packed as above (element pair (k, k+1) at byte
 *                       (k%128)/2, k in the low nibble).  Buffer:
 *                       round_up(rows, 2) * cols/2 bytes.
 *                       scales in 128-byte tiles of 32 rows x 4 blocks: the
 *                       byte of (row r, block b) is at
 *                       ((r/32)*(cols/128) + b/4)*128 + (r%32)*4 + b%4.
 *                       Buffer: round_up(rows, 32) * cols/32 bytes.
 *   One tiled scale tile is exactly what a 32x32x64 scaled MFMA operand
 *   needs per 32 rows and 128 K-elements, and one code tile feeds two rows
 *   of a 128-deep K stage, so the GEMM fetches whole cache lines.  Padding
 *   rows are never read.
 *   The GEMM operands A (activations, [M][K]) and B (packed weight, [N][K])
 *   are both MX_TILED, blocked along K.
 * - Arguments are checked on the host before anything is enqueued.  A
 *   status other than FP4DIT_OK means nothing was enqueued, except
 *   FP4DIT_E_LAUNCH, which reports a failed kernel launch.  No exception
 *   crosses the ABI; the only global state is a per-device cache of the CU
 *   count, kept in atomics, so calls from several host threads on different
 *   streams are safe.
 * - Zero-sized work (rows == 0, M == 0) returns FP4DIT_OK and enqueues
 *   nothing; the other sizes must still be valid.
 * - Every matrix size (rows, cols, M, N, K) must be below 2^31
 *   (FP4DIT_E_SHAPE otherwise); entry points state tighter limits where
 *   their kernels need them.
 *
 * Citations name the web pages this library implements: "fal" is the fal
 * page "Serving sub-second Ideogram v4 without quality loss" (FP4 execution
 * of a diffusion transformer with the post-GEMM ops fused into the GEMM
 * epilogue); "KroQuant" is the sns.style summary "KroQuant: efficient
 * post-training quantisation for diffusion transformers via Kronecker-product
 * structure".
 */
#ifndef FP4DIT_H
#define FP4DIT_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp4dit_status {
    FP4DIT_OK = 0,
    FP4DIT_E_NULL = 1,        /* a required pointer is NULL                     */
    FP4DIT_E_SHAPE = 2,       /* a size is negative, too large or not a needed multiple */
    FP4DIT_E_ALIGN = 3,       /* a pointer is not aligned as the entry point requires   */
    FP4DIT_E_UNSUPPORTED = 4, /* a dtype, head_dim or option combination not implemented */
    FP4DIT_E_LAUNCH = 5       /* the kernel launch failed (hipGetLastError)       */
} fp4dit_status;

typedef enum fp4dit_dtype {
    FP4DIT_F32 = 0,           /* IEEE binary32                                  */
    FP4DIT_BF16 = 1,          /* bfloat16 (uint16 bit patterns)                 */
    FP4DIT_F16 = 2            /* IEEE binary16 (sampler updates only)           */
} fp4dit_dtype;

typedef enum fp4dit_layout {
    FP4DIT_MX_ROWMAJOR = 0,   /* plain row-major codes and scales               */
    FP4DIT_MX_TILED = 1       /* 128-byte MFMA tiles (see above); GEMM operands */
} fp4dit_layout;

/* Human-readable name of a status code (static storage, never NULL). */
const char* fp4dit_status_string(fp4dit_status s);

/*
 * Online activation quantisation to MXFP4.
 * fal, "Running the transformer in FP4" (the 1-sign / 2-exponent / 1-mantissa
 * FP4 element); KroQuant, "Deep analysis" (W4A4 in MXFP4).
 *
 * x      [rows][cols] of x_dtype (F32 or BF16), 16-byte aligned.
 * codes, scales in `layout` (16-byte aligned codes); MX_TILED needs
 * cols % 128 == 0.
 * Per 32-element block: amax = max |x|; shared exponent
 * s = clamp(floor(log2 amax) - 2, -127, 127) (s = -127 for an all-zero
 * block); scale byte = s + 127; every element is x / 2^s rounded to the
 * nearest e2m1 magnitude, ties to even mantissa, saturating at 6, with the
 * sign bit of x (so -0 gives code 0x8).  A block holding Inf or NaN gets
 * scale byte 0xFF and zero codes.  Bit-exact: the result is unique.
 * Requires cols % 32 == 0.
 */
fp4dit_status fp4dit_quantize_mxfp4(const void* x, fp4dit_dtype x_dtype,
                                    int64_t rows, int64_t cols,
                                    uint8_t* codes, uint8_t* scales, fp4dit_layout layout,
                                    hipStream_t stream);

/*
 * Block-local transform of activations, optionally fused with MXFP4
 * quantisation of its result.
 * KroQuant, "Background and overview" (invertible transform on the
 * activations, inverse on the weights, applied online every step) and "Deep
 * analysis" (independent 32-element blocks, each with a learned matrix, run
 * as small-tile matrix-core GEMMs).
 *
 * y[r][32b + j] = sum_i x[r][32b + i] * T_b[i][j]   (y_b = x_b . T_b)
 * x       [rows][cols] of x_dtype (F32 or BF16), 16-byte aligned.
 * t_bf16  [n_t][32][32] bfloat16, row-major T_b[i][j]; n_t is 1 (one matrix
 *         for every block) or cols/32 (block b uses T_b).
 * y       NULL, or [rows][cols] of y_dtype (F32 or BF16, 16-byte aligned):
 *         the fp32 product, stored (BF16: round to nearest even).
 * codes, scales  both NULL, or both set: MXFP4 of the fp32 product exactly as
 *         fp4dit_quantize_mxfp4 would encode it, in `layout` (x never
 *         round-trips HBM).
 * At least one of y / codes must be set.  Products are exact and summed in
 * fp32: a BF16 x is the matrix-core operand itself; an F32 x is carried as
 * three bf16 parts (hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi -
 * mid)) whose sum is x exactly for |x| >= 2^-100 (below that, the part lost
 * is under 2^-133 in absolute value), so y is formed from the caller's
 * values and differs from x_b . T_b only by the order of the fp32 sums.
 * Requires cols % 32 == 0.
 */
fp4dit_status fp4dit_block_transform(const void* x, fp4dit_dtype x_dtype,
                                     int64_t rows, int64_t cols,
                                     const uint16_t* t_bf16, int64_t n_t,
                                     void* y, fp4dit_dtype y_dtype,
                                     uint8_t* codes, uint8_t* scales, fp4dit_layout layout,
                                     hipStream_t stream);

/*
 * Re-layout of an MXFP4 tensor (KroQuant, "Deep analysis": the W4A4 format
 * is MXFP4; fal, "Running the transformer in FP4": the e2m1 element) between
 * FP4DIT_MX_ROWMAJOR and FP4DIT_MX_TILED, in either direction (the same
 * layout on both sides is a copy).  Codes and scale bytes move; no value
 * changes, so the result is unique (bit-exact).  A caller holding the plain
 * row-major codes [rows][cols/2] and scales [rows][cols/32] gets the GEMM's
 * operand layout this way.
 *
 * in_codes, in_scales    [rows][cols] in in_layout (buffer sizes as the
 *                        layout states); out_codes, out_scales likewise in
 *                        out_layout.  The padding rows of a TILED output
 *                        (codes to round_up(rows, 2), scales to
 *                        round_up(rows, 32)) are written as zero.
 * cols % 128 == 0 if either side is TILED, else cols % 32 == 0; both codes
 * pointers 16-byte aligned; no output buffer may overlap an input buffer or
 * the other output (FP4DIT_E_UNSUPPORTED).
 */
fp4dit_status fp4dit_mx_relayout(const uint8_t* in_codes, const uint8_t* in_scales, fp4dit_layout in_layout,
                                 int64_t rows, int64_t cols, uint8_t* out_codes, uint8_t* out_scales,
                                 fp4dit_layout out_layout, hipStream_t stream);

/*
 * Offline weight side of the block transform: W'_b = T_b^-1 . W_b.
 * KroQuant, "Background and overview" (the inverse transform goes to the
 * weights).
 *
 * w      [K][N] float32, the logical weight of y = x . W; rows 32b..32b+31
 *        form block b.  w_out [K][N] float32 (may not alias w).
 * t_bf16, n_t as in fp4dit_block_transform (n_t is 1 or K/32).  Each block
 * is solved in fp64 by Gaussian elimination with partial pivoting and the
 * result rounded to fp32.  Returns FP4DIT_E_SHAPE unless K % 32 == 0.
 * A singular T_b gives non-finite w_out for that block.
 */
fp4dit_status fp4dit_fold_inverse_transform(const float* w, int64_t K, int64_t N,
                                            const uint16_t* t_bf16, int64_t n_t,
                                            float* w_out, hipStream_t stream);

/*
 * Offline weight packing: transpose the logical weight to [N][K] and quantise
 * it to MXFP4 along K (fal, "Running the transformer in FP4"; static FP4
 * weight quantisation for inference, QAD section).
 *
 * w      [K][N] of w_dtype (F32 or BF16), logical y = x . W.
 * codes, scales: the [N][K] MXFP4 weight in `layout` (MX_TILED for the GEMM).
 * interleave_group  0: no permutation.
 *        g > 0: SwiGLU weight (fal, "Fusing gated SiLU"): w holds
 *        [gate | up], N/2 columns each; physical column p takes logical
 *        output j = (p / 2g) * g + p % g from the up half if (p / g) is odd,
 *        else from the gate half, so gate and up outputs sit next to each
 *        other in the GEMM's output tile.  g must equal
 *        fp4dit_swiglu_interleave_group() for use with
 *        fp4dit_gemm_fp4_epilogue_swiglu, and N % (2g) == 0.
 * Same encoding as fp4dit_quantize_mxfp4.  Requires K % 32 == 0.
 */
fp4dit_status fp4dit_pack_weight(const void* w, fp4dit_dtype w_dtype,
                                 int64_t K, int64_t N, int32_t interleave_group,
                                 uint8_t* codes, uint8_t* scales, fp4dit_layout layout,
                                 hipStream_t stream);

/* Interleave group size g the SwiGLU epilogue expects (see fp4dit_pack_weight). */
int32_t fp4dit_swiglu_interleave_group(void);

/*
 * The GEMM shared by the three fused entry points below
 * (fal, section on epilogue fusion: A . B formed tile by tile with on-chip
 * fp32 accumulators; the epilogue runs before the one store to HBM):
 *     C[m][n] = sum_k D(A)[m][k] * D(B)[n][k]
 * with D() the exact MXFP4 value, scaled FP4 matrix-core products and fp32
 * accumulation.  A = (a_codes, a_scales) is [M][K] and B = (b_codes,
 * b_scales) is [N][K], both in the FP4DIT_MX_TILED layout (buffers padded
 * as stated there); every codes pointer 16-byte aligned, every scales
 * pointer 4-byte aligned.  Requires K % 128 == 0 and K >= 256 (the
 * 128-deep K stage, and the two stages the LDS ring's prologue loads),
 * N % 256 == 0 and N > 0, and M*K/2 and N*K/2 below 2^31 bytes; M >= 0 is
 * otherwise arbitrary (a ragged last token tile is masked).  The order of
 * the fp32 sums follows the launch's grid, which is derived from the
 * device's compute-unit count: on one device the same inputs give the same
 * bits on every call; devices with other CU counts may differ in the last
 * bits.
 */

/*
 * No epilogue: out [M][N] = C, stored as out_dtype (F32, or BF16 rounded to
 * nearest even).  out 16-byte aligned.  fal, epilogue-fusion section (cast).
 */
fp4dit_status fp4dit_gemm_fp4_epilogue_none(int64_t M, int64_t N, int64_t K,
                                            const uint8_t* a_codes, const uint8_t* a_scales,
                                            const uint8_t* b_codes, const uint8_t* b_scales,
                                            void* out, fp4dit_dtype out_dtype,
                                            hipStream_t stream);

/*
 * Per-head RMSNorm epilogue (fal, epilogue-fusion section and "Why
 * head_dim=256 is hard" / "Revisit fusion"): for every row and every head of
 * head_dim contiguous columns below n_norm_cols,
 *     y = C * rsqrt(mean(C^2 over the head) + eps) * norm_w[column],
 * with the statistics taken from the fp32 accumulators; columns at or past
 * n_norm_cols are stored unchanged (e.g. the V part of a fused QKV).
 * head_dim is 128 or 256; n_norm_cols % head_dim == 0, 0 <= n_norm_cols <= N;
 * norm_w [n_norm_cols] float32, 16-byte aligned (may be NULL only if
 * n_norm_cols == 0); eps >= 0 and finite.  out [M][N] of out_dtype,
 * 16-byte aligned.
 */
fp4dit_status fp4dit_gemm_fp4_epilogue_rmsnorm_head(int64_t M, int64_t N, int64_t K,
                                                    const uint8_t* a_codes, const uint8_t* a_scales,
                                                    const uint8_t* b_codes, const uint8_t* b_scales,
                                                    int32_t head_dim, int64_t n_norm_cols,
                                                    const float* norm_w, float eps,
                                                    void* out, fp4dit_dtype out_dtype,
                                                    hipStream_t stream);

/*
 * SwiGLU epilogue (fal, "Fusing gated SiLU"): with B packed by
 * fp4dit_pack_weight(..., fp4dit_swiglu_interleave_group(), ...) from
 * [gate | up], N physical columns give N/2 outputs
 *     h[m][j] = silu(gate[m][j]) * up[m][j],  silu(z) = z / (1 + exp(-z)).
 * out        NULL, or [M][N/2] of out_dtype (16-byte aligned).
 * out_codes, out_scales  both NULL, or both set: MXFP4 re-quantisation of
 *            the fp32 h [M][N/2] along its columns, in the MX_TILED layout
 *            (ready to be the A operand of the next GEMM; codes 16-byte,
 *            scales 2-byte aligned), encoded as fp4dit_quantize_mxfp4 does;
 *            both buffers below 2^31 bytes (else FP4DIT_E_SHAPE).
 * At least one output must be set.
 */
fp4dit_status fp4dit_gemm_fp4_epilogue_swiglu(int64_t M, int64_t N, int64_t K,
                                              const uint8_t* a_codes, const uint8_t* a_scales,
                                              const uint8_t* b_codes, const uint8_t* b_scales,
                                              void* out, fp4dit_dtype out_dtype,
                                              uint8_t* out_codes, uint8_t* out_scales,
                                              hipStream_t stream);

/*
 * SwiGLU epilogue carried through the next layer's block transform and
 * quantised (fal, "Fusing gated SiLU" and the epilogue-fusion section: the
 * output makes no HBM round trip; KroQuant, "Background and overview" and
 * "Deep analysis": the down projection's input is transformed per 32-element
 * block before it is quantised).  With h [M][N/2] as in
 * fp4dit_gemm_fp4_epilogue_swiglu (same B packing and constraints on N):
 *     y[m][32b + j] = sum_i h[m][32b + i] * T_b[i][j]
 * computed from the fp32 h (not a bf16 copy of it: h is carried exactly as
 * three bf16 parts, as an F32 x in fp4dit_block_transform, and the products
 * are summed in fp32), then MXFP4-quantised along its columns.
 * t_bf16     [n_t][32][32] bfloat16 bit patterns, row i = input feature,
 *            2-byte aligned; n_t = 1 (one T for every block) or N/64.
 * y          NULL, or [M][N/2] of y_dtype (16-byte aligned): y itself.
 * out_codes, out_scales  required: MXFP4 codes / scales of y in the
 *            MX_TILED layout (codes 16-byte, scales 2-byte aligned), ready
 *            to be the A operand of the down-projection GEMM, whose weights
 *            carry the inverse transform (fp4dit_fold_inverse_transform);
 *            both below 2^31 bytes (else FP4DIT_E_SHAPE).
 */
fp4dit_status fp4dit_gemm_fp4_epilogue_swiglu_transform(int64_t M, int64_t N, int64_t K,
                                                        const uint8_t* a_codes, const uint8_t* a_scales,
                                                        const uint8_t* b_codes, const uint8_t* b_scales,
                                                        const uint16_t* t_bf16, int64_t n_t,
                                                        void* y, fp4dit_dtype y_dtype,
                                                        uint8_t* out_codes, uint8_t* out_scales,
                                                        hipStream_t stream);

/*
 * Unfused epilogues.  fal, "Epilogue fusion in brief": without fusion the
 * GEMM's output makes a round trip through HBM and each small op is a launch
 * of its own.  These two calls are those launches, on a bf16 GEMM output
 * (fp4dit_gemm_fp4_epilogue_none with out_dtype BF16); they exist to measure
 * what the fused epilogues save, and compute the same definitions on the
 * bf16 values, in fp32, with a bf16 (round to nearest even) result.
 *
 * Per-head RMSNorm, as fp4dit_gemm_fp4_epilogue_rmsnorm_head: x and out
 * [rows][cols] bf16 bit patterns (out may equal x), 16-byte aligned;
 * head_dim 128 or 256 with cols % head_dim == 0; n_norm_cols % head_dim
 * == 0 and <= cols; norm_w [n_norm_cols] float32, 16-byte aligned (may be
 * NULL only if n_norm_cols == 0); eps >= 0 and finite; rows * cols / 8
 * below 2^32.
 */
fp4dit_status fp4dit_rmsnorm_head(const uint16_t* x, int64_t rows, int64_t cols, int32_t head_dim,
                                  int64_t n_norm_cols, const float* norm_w, float eps, uint16_t* out,
                                  hipStream_t stream);

/*
 * SwiGLU, as fp4dit_gemm_fp4_epilogue_swiglu, over c [rows][n_phys] bf16
 * whose columns are interleaved with group g (fp4dit_pack_weight's
 * interleave_group): h [rows][n_phys/2] bf16 = silu(gate) * up.  g % 8 == 0,
 * n_phys % (2g) == 0, rows * n_phys / 16 below 2^32; c and h 16-byte
 * aligned and not overlapping (else FP4DIT_E_UNSUPPORTED).
 */
fp4dit_status fp4dit_swiglu(const uint16_t* c, int64_t rows, int64_t n_phys, int32_t group, uint16_t* h,
                            hipStream_t stream);

/*
 * QAD fake quantisation (fal, QAD section: the student's forward pass goes
 * through its own FP4 rounding, so the quantisation noise propagates; the
 * backward pass routes the gradient around the rounding with a
 * straight-through estimator, i.e. dL/dx = dL/dy, which needs no kernel).
 * y = D(Q(x)): every 32-element block of a row is quantised exactly as
 * fp4dit_quantize_mxfp4 does and each code is replaced by its value,
 * level * 2^s.  Those values are exact in F32 and in BF16, so the result is
 * unique (bit-exact, -0 for code 0x8); a block holding Inf or NaN gives NaN.
 * x [rows][cols] of x_dtype, y [rows][cols] of y_dtype (F32 or BF16 each),
 * both 16-byte aligned; y may equal x when the dtypes match; cols % 32 == 0.
 */
fp4dit_status fp4dit_fake_quantize_mxfp4(const void* x, fp4dit_dtype x_dtype, int64_t rows, int64_t cols,
                                         void* y, fp4dit_dtype y_dtype, hipStream_t stream);

/*
 * Diffusion-sampler updates ("拡散サンプリングの高速化：数値計算手法と
 * スコアベースモデルの出会い", sections on the exponential integrator, on
 * Richardson extrapolation and on the fused update kernels), elementwise over
 * n elements of one dtype (F32, BF16 or F16; every pointer 16-byte aligned;
 * out may equal an input but not overlap one otherwise), computed in fp32
 * and rounded once (to nearest even) into the dtype:
 *   ETD1        out = decay * x + coeff * x0
 *   ETD2        out = decay * x + c0 * x0 + c1 * x0_prev
 *   Richardson  out = (scale * fine - coarse) / (scale - 1), scale != 1
 * x is the current state, x0 / x0_prev the network's data predictions at
 * this step and the previous one, fine / coarse the results of an order-p
 * method with 2N and N steps (scale = 2^p).  n < 2^40.
 */
fp4dit_status fp4dit_etd1_update(const void* x, const void* x0, int64_t n, fp4dit_dtype dtype, float decay,
                                 float coeff, void* out, hipStream_t stream);
fp4dit_status fp4dit_etd2_update(const void* x, const void* x0, const void* x0_prev, int64_t n,
                                 fp4dit_dtype dtype, float decay, float c0, float c1, void* out,
                                 hipStream_t stream);
fp4dit_status fp4dit_richardson_combine(const void* fine, const void* coarse, int64_t n, fp4dit_dtype dtype,
                                        float scale, void* out, hipStream_t stream);

/*
 * Host-only: the scalars of one ETD step from schedule point (alpha_s,
 * sigma_s) to (alpha_t, sigma_t), all > 0, with h = lambda_t - lambda_s and
 * lambda = log(alpha / sigma) (same page, exponential-integrator section):
 *   decay = e^-h * alpha_t / alpha_s,  coeff = alpha_t * (1 - e^-h),
 * the coefficients that make the step exact for a data prediction held
 * constant over it.  order 1 (ETD1): c0 = coeff, c1 = 0.  order 2 (ETD2):
 * c0 = 3/4 coeff, c1 = 1/4 coeff, except on the first step (first_step != 0),
 * which has no previous prediction and is ETD1.  Computed in double.
 * Returns FP4DIT_E_UNSUPPORTED for another order, FP4DIT_E_SHAPE for a
 * non-positive or non-finite schedule value, FP4DIT_E_NULL for a NULL output.
 */
fp4dit_status fp4dit_etd_coefficients(double alpha_s, double sigma_s, double alpha_t, double sigma_t,
                                      int32_t order, int32_t first_step, double* decay, double* c0,
                                      double* c1);

#ifdef __cplusplus
}
#endif

#endif /* FP4DIT_H */
