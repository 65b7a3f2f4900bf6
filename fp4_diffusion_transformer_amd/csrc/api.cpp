// C ABI of libfp4dit.so (declared in include/fp4dit.h): host-side argument
// validation, then the launch on the caller's stream.  Validation never
// dereferences a pointer and runs before any HIP call, so a non-OK status
// other than FP4DIT_E_LAUNCH means nothing was enqueued.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "../../include/fp4dit.h"
#include "launch.hpp"

namespace {

using fp4dit::kGemmKMin;
using fp4dit::kGemmKMultiple;
using fp4dit::kGemmNMultiple;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_dtype(fp4dit_dtype d) { return d == FP4DIT_F32 || d == FP4DIT_BF16; }
bool valid_sampler_dtype(fp4dit_dtype d) { return d == FP4DIT_F32 || d == FP4DIT_BF16 || d == FP4DIT_F16; }
int dtype_bytes(fp4dit_dtype d) { return d == FP4DIT_F32 ? 4 : 2; }
// out may be one of the inputs (same start), or else must not overlap it.
bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x != y && x < y + uintptr_t(b_bytes) && y < x + uintptr_t(a_bytes);
}
bool valid_layout(fp4dit_layout l) { return l == FP4DIT_MX_ROWMAJOR || l == FP4DIT_MX_TILED; }
fp4dit_status launched(hipError_t e) { return e == hipSuccess ? FP4DIT_OK : FP4DIT_E_LAUNCH; }

// Every matrix size is below 2^31, so a product of two sizes (times a few
// bytes) fits in int64 before the finer limits below are checked.
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
bool dims_ok(std::initializer_list<int64_t> dims) {
    for (int64_t d : dims)
        if (d > kMaxDim) return false;
    return true;
}

// Byte offsets inside the GEMM operands are 32-bit (tiled buffers are padded
// to an even number of rows).
constexpr int64_t kMaxOperandBytes = (int64_t(1) << 31) - 1;

// The requant epilogue forms its output offsets in 32 bits.
bool requant_fits(int64_t M, int64_t N) {
    return (M + 1) * (N / 4) <= kMaxOperandBytes && (M + 31) * (N / 64) <= kMaxOperandBytes;
}

fp4dit_status check_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                         const uint8_t* bc, const uint8_t* bs) {
    if (M < 0 || N <= 0 || K <= 0 || !dims_ok({M, N, K})) return FP4DIT_E_SHAPE;
    if (N % kGemmNMultiple != 0 || K % kGemmKMultiple != 0 || K < kGemmKMin) return FP4DIT_E_SHAPE;
    if ((M + 1) * (K / 2) > kMaxOperandBytes || N * (K / 2) > kMaxOperandBytes) return FP4DIT_E_SHAPE;
    if (M == 0) return FP4DIT_OK;
    if (!ac || !as || !bc || !bs) return FP4DIT_E_NULL;
    if (!aligned(ac, 16) || !aligned(bc, 16) || !aligned(as, 4) || !aligned(bs, 4)) return FP4DIT_E_ALIGN;
    return FP4DIT_OK;
}

}  // namespace

extern "C" {

const char* fp4dit_status_string(fp4dit_status s) {
    switch (s) {
        case FP4DIT_OK: return "ok";
        case FP4DIT_E_NULL: return "null pointer";
        case FP4DIT_E_SHAPE: return "invalid shape";
        case FP4DIT_E_ALIGN: return "misaligned pointer";
        case FP4DIT_E_UNSUPPORTED: return "unsupported argument";
        case FP4DIT_E_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int32_t fp4dit_swiglu_interleave_group(void) { return fp4dit::kSwigluGroup; }

fp4dit_status fp4dit_quantize_mxfp4(const void* x, fp4dit_dtype x_dtype, int64_t rows, int64_t cols,
                                    uint8_t* codes, uint8_t* scales, fp4dit_layout layout, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_layout(layout)) return FP4DIT_E_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % (layout == FP4DIT_MX_TILED ? 128 : 32) != 0) return FP4DIT_E_SHAPE;
    if (!dims_ok({rows, cols})) return FP4DIT_E_SHAPE;
    if (rows == 0 || cols == 0) return FP4DIT_OK;
    if (rows * (cols / 32) >= (int64_t(1) << 32)) return FP4DIT_E_SHAPE;
    if (!x || !codes || !scales) return FP4DIT_E_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_quantize(x, x_dtype == FP4DIT_BF16, rows, cols, codes, scales,
                                            layout == FP4DIT_MX_TILED, stream));
}

fp4dit_status fp4dit_block_transform(const void* x, fp4dit_dtype x_dtype, int64_t rows, int64_t cols,
                                     const uint16_t* t_bf16, int64_t n_t, void* y, fp4dit_dtype y_dtype,
                                     uint8_t* codes, uint8_t* scales, fp4dit_layout layout, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || (y && !valid_dtype(y_dtype))) return FP4DIT_E_UNSUPPORTED;
    if ((codes == nullptr) != (scales == nullptr)) return FP4DIT_E_UNSUPPORTED;
    if (codes && !valid_layout(layout)) return FP4DIT_E_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 32 != 0 || !dims_ok({rows, cols})) return FP4DIT_E_SHAPE;
    if (codes && layout == FP4DIT_MX_TILED && cols % 128 != 0) return FP4DIT_E_SHAPE;
    if (n_t != 1 && n_t != cols / 32) return FP4DIT_E_SHAPE;
    if (rows == 0 || cols == 0) return FP4DIT_OK;
    if (cols / 32 > (int64_t(1) << 20) || rows > (int64_t(1) << 23)) return FP4DIT_E_SHAPE;  // grid.y <= 65535
    if (!x || !t_bf16) return FP4DIT_E_NULL;
    if (!y && !codes) return FP4DIT_E_NULL;
    if (!aligned(x, 16) || !aligned(t_bf16, 2) || (y && !aligned(y, 16)) || (codes && !aligned(codes, 16)))
        return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_block_transform(x, x_dtype == FP4DIT_BF16, rows, cols, t_bf16, n_t, y,
                                                   y_dtype == FP4DIT_BF16, codes, scales,
                                                   layout == FP4DIT_MX_TILED, stream));
}

fp4dit_status fp4dit_fold_inverse_transform(const float* w, int64_t K, int64_t N, const uint16_t* t_bf16,
                                            int64_t n_t, float* w_out, hipStream_t stream) {
    if (K < 0 || N < 0 || K % 32 != 0 || !dims_ok({K, N})) return FP4DIT_E_SHAPE;
    if (n_t != 1 && n_t != K / 32) return FP4DIT_E_SHAPE;
    if (K == 0 || N == 0) return FP4DIT_OK;
    if (K / 32 > 65535) return FP4DIT_E_SHAPE;
    if (!w || !t_bf16 || !w_out) return FP4DIT_E_NULL;
    if (w == w_out) return FP4DIT_E_UNSUPPORTED;
    if (!aligned(w, 4) || !aligned(w_out, 4) || !aligned(t_bf16, 2)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_fold_inverse(w, K, N, t_bf16, n_t, w_out, stream));
}

fp4dit_status fp4dit_mx_relayout(const uint8_t* in_codes, const uint8_t* in_scales, fp4dit_layout in_layout,
                                 int64_t rows, int64_t cols, uint8_t* out_codes, uint8_t* out_scales,
                                 fp4dit_layout out_layout, hipStream_t stream) {
    if (!valid_layout(in_layout) || !valid_layout(out_layout)) return FP4DIT_E_UNSUPPORTED;
    const bool tiled = in_layout == FP4DIT_MX_TILED || out_layout == FP4DIT_MX_TILED;
    if (rows < 0 || cols < 0 || cols % (tiled ? 128 : 32) != 0 || !dims_ok({rows, cols})) return FP4DIT_E_SHAPE;
    if (rows == 0 || cols == 0) return FP4DIT_OK;
    if (!in_codes || !in_scales || !out_codes || !out_scales) return FP4DIT_E_NULL;
    if (!aligned(in_codes, 16) || !aligned(out_codes, 16)) return FP4DIT_E_ALIGN;
    auto code_bytes = [&](fp4dit_layout l) { return (l == FP4DIT_MX_TILED ? (rows + 1) / 2 * 2 : rows) * (cols / 2); };
    auto scale_bytes = [&](fp4dit_layout l) {
        return (l == FP4DIT_MX_TILED ? (rows + 31) / 32 * 32 : rows) * (cols / 32);
    };
    const void* ins[2] = {in_codes, in_scales};
    const int64_t in_b[2] = {code_bytes(in_layout), scale_bytes(in_layout)};
    const void* outs[2] = {out_codes, out_scales};
    const int64_t out_b[2] = {code_bytes(out_layout), scale_bytes(out_layout)};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            if (outs[i] == ins[j] || overlaps(outs[i], out_b[i], ins[j], in_b[j])) return FP4DIT_E_UNSUPPORTED;
    if (outs[0] == outs[1] || overlaps(outs[0], out_b[0], outs[1], out_b[1])) return FP4DIT_E_UNSUPPORTED;
    return launched(fp4dit::launch_relayout(in_codes, in_scales, in_layout == FP4DIT_MX_TILED, rows, cols, out_codes,
                                            out_scales, out_layout == FP4DIT_MX_TILED, stream));
}

fp4dit_status fp4dit_pack_weight(const void* w, fp4dit_dtype w_dtype, int64_t K, int64_t N,
                                 int32_t interleave_group, uint8_t* codes, uint8_t* scales,
                                 fp4dit_layout layout, hipStream_t stream) {
    if (!valid_dtype(w_dtype) || !valid_layout(layout)) return FP4DIT_E_UNSUPPORTED;
    if (interleave_group < 0) return FP4DIT_E_UNSUPPORTED;
    if (K < 0 || N < 0 || K % (layout == FP4DIT_MX_TILED ? 128 : 32) != 0) return FP4DIT_E_SHAPE;
    if (!dims_ok({K, N})) return FP4DIT_E_SHAPE;
    if (interleave_group > 0 && N % (2 * (int64_t)interleave_group) != 0) return FP4DIT_E_SHAPE;
    if (K == 0 || N == 0) return FP4DIT_OK;
    if (K / 32 > 65535) return FP4DIT_E_SHAPE;
    if (!w || !codes || !scales) return FP4DIT_E_NULL;
    if (!aligned(codes, 16) || !aligned(w, w_dtype == FP4DIT_BF16 ? 2 : 4)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_pack_weight(w, w_dtype == FP4DIT_BF16, K, N, interleave_group, codes,
                                               scales, layout == FP4DIT_MX_TILED, stream));
}

fp4dit_status fp4dit_gemm_fp4_epilogue_none(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                            const uint8_t* a_scales, const uint8_t* b_codes,
                                            const uint8_t* b_scales, void* out, fp4dit_dtype out_dtype,
                                            hipStream_t stream) {
    if (!valid_dtype(out_dtype)) return FP4DIT_E_UNSUPPORTED;
    const fp4dit_status st = check_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales);
    if (st != FP4DIT_OK || M == 0) return st;
    if (!out) return FP4DIT_E_NULL;
    if (!aligned(out, 16)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_gemm_none(M, N, K, a_codes, a_scales, b_codes, b_scales, out,
                                             out_dtype == FP4DIT_BF16, stream));
}

fp4dit_status fp4dit_gemm_fp4_epilogue_rmsnorm_head(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                                    const uint8_t* a_scales, const uint8_t* b_codes,
                                                    const uint8_t* b_scales, int32_t head_dim,
                                                    int64_t n_norm_cols, const float* norm_w, float eps,
                                                    void* out, fp4dit_dtype out_dtype, hipStream_t stream) {
    if (!valid_dtype(out_dtype)) return FP4DIT_E_UNSUPPORTED;
    if (head_dim != 128 && head_dim != 256) return FP4DIT_E_UNSUPPORTED;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return FP4DIT_E_UNSUPPORTED;
    const fp4dit_status st = check_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales);
    if (st != FP4DIT_OK) return st;
    if (n_norm_cols < 0 || n_norm_cols > N || n_norm_cols % head_dim != 0) return FP4DIT_E_SHAPE;
    if (M == 0) return FP4DIT_OK;
    if (!out || (n_norm_cols > 0 && !norm_w)) return FP4DIT_E_NULL;
    if (!aligned(out, 16) || (n_norm_cols > 0 && !aligned(norm_w, 16))) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_gemm_rmsnorm(M, N, K, a_codes, a_scales, b_codes, b_scales, head_dim,
                                                n_norm_cols, norm_w, eps, out, out_dtype == FP4DIT_BF16,
                                                stream));
}

fp4dit_status fp4dit_gemm_fp4_epilogue_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                              const uint8_t* a_scales, const uint8_t* b_codes,
                                              const uint8_t* b_scales, void* out, fp4dit_dtype out_dtype,
                                              uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream) {
    if (out && !valid_dtype(out_dtype)) return FP4DIT_E_UNSUPPORTED;
    if ((out_codes == nullptr) != (out_scales == nullptr)) return FP4DIT_E_UNSUPPORTED;
    const fp4dit_status st = check_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales);
    if (st != FP4DIT_OK) return st;
    if (N % (2 * fp4dit::kSwigluGroup) != 0) return FP4DIT_E_SHAPE;
    if (out_codes && !requant_fits(M, N)) return FP4DIT_E_SHAPE;
    if (M == 0) return FP4DIT_OK;
    if (!out && !out_codes) return FP4DIT_E_NULL;
    if ((out && !aligned(out, 16)) || (out_codes && (!aligned(out_codes, 16) || !aligned(out_scales, 2))))
        return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_gemm_swiglu(M, N, K, a_codes, a_scales, b_codes, b_scales, out,
                                               out_dtype == FP4DIT_BF16, out_codes, out_scales, stream));
}

fp4dit_status fp4dit_gemm_fp4_epilogue_swiglu_transform(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                                        const uint8_t* a_scales, const uint8_t* b_codes,
                                                        const uint8_t* b_scales, const uint16_t* t_bf16,
                                                        int64_t n_t, void* y, fp4dit_dtype y_dtype,
                                                        uint8_t* out_codes, uint8_t* out_scales,
                                                        hipStream_t stream) {
    if (y && !valid_dtype(y_dtype)) return FP4DIT_E_UNSUPPORTED;
    const fp4dit_status st = check_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales);
    if (st != FP4DIT_OK) return st;
    if (N % (2 * fp4dit::kSwigluGroup) != 0) return FP4DIT_E_SHAPE;
    if (n_t != 1 && n_t != N / 64) return FP4DIT_E_SHAPE;
    if (!requant_fits(M, N)) return FP4DIT_E_SHAPE;
    if (M == 0) return FP4DIT_OK;
    if (!t_bf16 || !out_codes || !out_scales) return FP4DIT_E_NULL;
    if ((y && !aligned(y, 16)) || !aligned(t_bf16, 2) || !aligned(out_codes, 16) || !aligned(out_scales, 2))
        return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_gemm_swiglu_transform(M, N, K, a_codes, a_scales, b_codes, b_scales, t_bf16,
                                                         n_t, y, y_dtype == FP4DIT_BF16, out_codes, out_scales,
                                                         stream));
}

fp4dit_status fp4dit_rmsnorm_head(const uint16_t* x, int64_t rows, int64_t cols, int32_t head_dim,
                                  int64_t n_norm_cols, const float* norm_w, float eps, uint16_t* out,
                                  hipStream_t stream) {
    if (head_dim != 128 && head_dim != 256) return FP4DIT_E_UNSUPPORTED;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return FP4DIT_E_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % head_dim != 0 || !dims_ok({rows, cols})) return FP4DIT_E_SHAPE;
    if (n_norm_cols < 0 || n_norm_cols > cols || n_norm_cols % head_dim != 0) return FP4DIT_E_SHAPE;
    if (rows == 0 || cols == 0) return FP4DIT_OK;
    if (rows * (cols / 8) >= (int64_t(1) << 32)) return FP4DIT_E_SHAPE;
    if (!x || !out || (n_norm_cols > 0 && !norm_w)) return FP4DIT_E_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || (norm_w && !aligned(norm_w, 16))) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_rmsnorm_head(x, rows, cols, head_dim, n_norm_cols, norm_w, eps, out, stream));
}

fp4dit_status fp4dit_swiglu(const uint16_t* c, int64_t rows, int64_t n_phys, int32_t group, uint16_t* h,
                            hipStream_t stream) {
    if (group <= 0 || group % 8 != 0) return FP4DIT_E_UNSUPPORTED;
    if (rows < 0 || n_phys < 0 || n_phys % (2 * int64_t(group)) != 0 || !dims_ok({rows, n_phys}))
        return FP4DIT_E_SHAPE;
    if (rows == 0 || n_phys == 0) return FP4DIT_OK;
    if (rows * (n_phys / 16) >= (int64_t(1) << 32)) return FP4DIT_E_SHAPE;
    if (!c || !h) return FP4DIT_E_NULL;
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(c), h0 = reinterpret_cast<uintptr_t>(h);
    if (h0 < c0 + uintptr_t(rows * n_phys * 2) && c0 < h0 + uintptr_t(rows * n_phys)) return FP4DIT_E_UNSUPPORTED;
    if (!aligned(c, 16) || !aligned(h, 16)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_swiglu(c, rows, n_phys, group, h, stream));
}

fp4dit_status fp4dit_fake_quantize_mxfp4(const void* x, fp4dit_dtype x_dtype, int64_t rows, int64_t cols,
                                         void* y, fp4dit_dtype y_dtype, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return FP4DIT_E_UNSUPPORTED;
    if (rows < 0 || cols < 0 || cols % 32 != 0 || !dims_ok({rows, cols})) return FP4DIT_E_SHAPE;
    if (rows == 0 || cols == 0) return FP4DIT_OK;
    if (rows * (cols / 8) >= (int64_t(1) << 40)) return FP4DIT_E_SHAPE;
    if (!x || !y) return FP4DIT_E_NULL;
    if (x == y && x_dtype != y_dtype) return FP4DIT_E_UNSUPPORTED;
    if (overlaps(x, rows * cols * dtype_bytes(x_dtype), y, rows * cols * dtype_bytes(y_dtype)))
        return FP4DIT_E_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(y, 16)) return FP4DIT_E_ALIGN;
    return launched(fp4dit::launch_fake_quant(x, x_dtype == FP4DIT_BF16, rows, cols, y, y_dtype == FP4DIT_BF16,
                                              stream));
}

namespace {
fp4dit_status check_sampler(const void* const* in, int n_in, int64_t n, fp4dit_dtype dtype, const void* out) {
    if (!valid_sampler_dtype(dtype)) return FP4DIT_E_UNSUPPORTED;
    if (n < 0 || n >= (int64_t(1) << 40)) return FP4DIT_E_SHAPE;
    if (n == 0) return FP4DIT_OK;
    if (!out) return FP4DIT_E_NULL;
    for (int i = 0; i < n_in; ++i)
        if (!in[i]) return FP4DIT_E_NULL;
    for (int i = 0; i < n_in; ++i)
        if (overlaps(in[i], n * dtype_bytes(dtype), out, n * dtype_bytes(dtype))) return FP4DIT_E_UNSUPPORTED;
    if (!aligned(out, 16)) return FP4DIT_E_ALIGN;
    for (int i = 0; i < n_in; ++i)
        if (!aligned(in[i], 16)) return FP4DIT_E_ALIGN;
    return FP4DIT_OK;
}
}  // namespace

fp4dit_status fp4dit_etd1_update(const void* x, const void* x0, int64_t n, fp4dit_dtype dtype, float decay,
                                 float coeff, void* out, hipStream_t stream) {
    const void* in[2] = {x, x0};
    const fp4dit_status st = check_sampler(in, 2, n, dtype, out);
    if (st != FP4DIT_OK || n == 0) return st;
    return launched(fp4dit::launch_etd1(x, x0, n, (int)dtype, decay, coeff, out, stream));
}

fp4dit_status fp4dit_etd2_update(const void* x, const void* x0, const void* x0_prev, int64_t n,
                                 fp4dit_dtype dtype, float decay, float c0, float c1, void* out,
                                 hipStream_t stream) {
    const void* in[3] = {x, x0, x0_prev};
    const fp4dit_status st = check_sampler(in, 3, n, dtype, out);
    if (st != FP4DIT_OK || n == 0) return st;
    return launched(fp4dit::launch_etd2(x, x0, x0_prev, n, (int)dtype, decay, c0, c1, out, stream));
}

fp4dit_status fp4dit_richardson_combine(const void* fine, const void* coarse, int64_t n, fp4dit_dtype dtype,
                                        float scale, void* out, hipStream_t stream) {
    if (!(scale != 1.0f) || !std::isfinite(scale)) return FP4DIT_E_UNSUPPORTED;
    const void* in[2] = {fine, coarse};
    const fp4dit_status st = check_sampler(in, 2, n, dtype, out);
    if (st != FP4DIT_OK || n == 0) return st;
    return launched(fp4dit::launch_richardson(fine, coarse, n, (int)dtype, scale, out, stream));
}

fp4dit_status fp4dit_etd_coefficients(double alpha_s, double sigma_s, double alpha_t, double sigma_t,
                                      int32_t order, int32_t first_step, double* decay, double* c0,
                                      double* c1) {
    if (order != 1 && order != 2) return FP4DIT_E_UNSUPPORTED;
    const double v[4] = {alpha_s, sigma_s, alpha_t, sigma_t};
    for (double a : v)
        if (!(a > 0.0) || !std::isfinite(a)) return FP4DIT_E_SHAPE;
    if (!decay || !c0 || !c1) return FP4DIT_E_NULL;
    const double h = std::log(alpha_t / sigma_t) - std::log(alpha_s / sigma_s);
    const double e = std::exp(-h);
    const double coeff = alpha_t * (1.0 - e);
    *decay = e * alpha_t / alpha_s;
    if (order == 1 || first_step) {
        *c0 = coeff;
        *c1 = 0.0;
    } else {
        *c0 = 0.75 * coeff;
        *c1 = 0.25 * coeff;
    }
    return FP4DIT_OK;
}

}  // extern "C"
