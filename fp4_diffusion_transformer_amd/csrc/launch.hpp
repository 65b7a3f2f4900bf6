// Internal launchers of the fp4dit kernels, called by the C ABI layer after
// argument validation.  Each enqueues on `stream` and returns
// hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dit {

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream);

hipError_t launch_pack_weight(const void* w, bool bf16, int64_t K, int64_t N, int group,
                              uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream);

hipError_t launch_block_transform(const void* x, bool x_bf16, int64_t rows, int64_t cols,
                                  const uint16_t* t, int64_t n_t, void* y, bool y_bf16,
                                  uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream);

hipError_t launch_relayout(const uint8_t* in_codes, const uint8_t* in_scales, bool in_tiled, int64_t rows,
                           int64_t cols, uint8_t* out_codes, uint8_t* out_scales, bool out_tiled,
                           hipStream_t stream);

hipError_t launch_fold_inverse(const float* w, int64_t K, int64_t N, const uint16_t* t, int64_t n_t,
                               float* w_out, hipStream_t stream);

hipError_t launch_gemm_none(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                            const uint8_t* bc, const uint8_t* bs, void* out, bool out_bf16,
                            hipStream_t stream);

hipError_t launch_gemm_rmsnorm(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                               const uint8_t* bc, const uint8_t* bs, int head_dim, int64_t n_norm,
                               const float* norm_w, float eps, void* out, bool out_bf16,
                               hipStream_t stream);

hipError_t launch_gemm_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                              const uint8_t* bc, const uint8_t* bs, void* out, bool out_bf16,
                              uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream);

hipError_t launch_gemm_swiglu_transform(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                                        const uint8_t* bc, const uint8_t* bs, const uint16_t* t, int64_t n_t,
                                        void* out, bool out_bf16, uint8_t* out_codes, uint8_t* out_scales,
                                        hipStream_t stream);

hipError_t launch_rmsnorm_head(const uint16_t* x, int64_t rows, int64_t cols, int head_dim, int64_t n_norm,
                               const float* w, float eps, uint16_t* y, hipStream_t stream);

hipError_t launch_swiglu(const uint16_t* c, int64_t rows, int64_t n_phys, int group, uint16_t* h,
                         hipStream_t stream);

hipError_t launch_fake_quant(const void* x, bool x_bf16, int64_t rows, int64_t cols, void* y, bool y_bf16,
                             hipStream_t stream);

// Sampler updates; storage: 0 fp32, 1 bf16, 2 fp16 (the fp4dit_dtype values).
hipError_t launch_etd1(const void* x, const void* x0, int64_t n, int storage, float decay, float coeff, void* out,
                       hipStream_t stream);
hipError_t launch_etd2(const void* x, const void* x0, const void* x0_prev, int64_t n, int storage, float decay,
                       float c0, float c1, void* out, hipStream_t stream);
hipError_t launch_richardson(const void* fine, const void* coarse, int64_t n, int storage, float scale, void* out,
                             hipStream_t stream);

// Interleave group of the SwiGLU epilogue: channel blocks of 32 alternate
// gate / up, matching one 32x32 MFMA output block per half.
constexpr int kSwigluGroup = 32;
// GEMM tiling constraints checked by the ABI layer: N a multiple of the
// 256-channel tile; K a multiple of the 128-deep LDS stage, and at least the
// two stages the ring's prologue loads.
constexpr int64_t kGemmNMultiple = 256;
constexpr int64_t kGemmKMultiple = 128;
constexpr int64_t kGemmKMin = 256;

}  // namespace fp4dit
