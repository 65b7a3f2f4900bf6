// Block-local activation transform (optionally fused with MXFP4 quantise)
// and its offline weight-side inverse.
//
// KroQuant, "Background and overview": an invertible linear transform
// smooths the activations and its inverse goes to the weights; it runs online
// every denoising step, so its cost matters.  "Deep analysis": the
// activations are split into independent 32-element blocks with one learned
// matrix each, which turns the transform into small-tile matrix-core GEMMs.
//
// Online kernel (HBM-bound): one wave owns 4 consecutive blocks (128
// channels) of 4 x 32 tokens; each 32-token group is staged in LDS by
// direct-to-LDS loads of whole rows (double-buffered, see issue_group).  Per
// block it runs two bf16 MFMAs V_MFMA_F32_32X32X16_BF16 (six for an fp32 x,
// carried as three bf16 parts) computing Y_b^T = T_b^T . X_b^T, i.e. lane l
// ends with token l%32 and output features 8a + 4(l/32) + r (a, r = 0..3) --
// the same accumulator layout as the GEMM epilogue, so the fused MXFP4
// encoding is shared with it: the block amax is one in-lane max plus one
// lane-swap (v_permlane32_swap).
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

typedef short v8s __attribute__((ext_vector_type(8)));

// Encode one 32-wide block of an MFMA 32x32 accumulator row (this lane's 16
// values hv[4a + r] = feature 8a + 4h + r) to MXFP4 and store it.
__device__ __forceinline__ void store_mx_block(const float* hv, int lane, bool live,
                                               uint8_t* codes16, uint8_t* scale1) {
    const int h = lane >> 5;
    const uint32_t amax = max_xor32_u(amax_bits<16>(hv));
    const uint32_t sc = e8m0_from_amax_bits(amax);
    uint32_t c16[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) c16[a] = sc == 0xFFu ? 0u : e2m1_pack4(hv + 4 * a, sc);
    const uint32_t send = h == 0 ? (c16[2] | (c16[3] << 16)) : (c16[0] | (c16[1] << 16));
    const uint32_t recv = partner_xor32(send, lane);
    v2u st;
    if (h == 0) {
        st[0] = c16[0] | ((recv & 0xFFFFu) << 16);
        st[1] = c16[1] | ((recv >> 16) << 16);
    } else {
        st[0] = (recv & 0xFFFFu) | (c16[2] << 16);
        st[1] = (recv >> 16) | (c16[3] << 16);
    }
    if (live) {
        *reinterpret_cast<v2u*>(codes16 + h * 8) = st;
        if (h == 0) *scale1 = (uint8_t)sc;
    }
}

constexpr int kTokIters = 4;           // 32-token groups per wave

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding): vmcnt, expcnt, lgkmcnt.
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
    return (vm & 15) | ((exp & 7) << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

// Loads of a 32-token group: each wave stages its 32 tokens x 128 channels
// (4 blocks) in its own LDS buffer with direct-to-LDS loads.  One load moves
// 64 x 16 B = whole rows (4 of bf16, 2 of fp32), i.e. full cache lines; in
// LDS the 16-byte chunk c of row r sits at c ^ (r & 15), so that the operand
// reads below (lane = token row, fixed chunk) hit 16 different chunk
// positions per quarter-wave: no bank conflicts.  Rows past the last token
// and chunks past the last column are clamped to valid memory (never used).
template <int kEsz>
__device__ __forceinline__ void issue_group(uint8_t* buf, const void* x, int64_t rows, int64_t cols,
                                            int64_t tok0, int64_t b0, int lane) {
    constexpr int kChunks = 128 * kEsz / 16;             // 16-byte chunks per token row
    constexpr int kLoads = 32 * kChunks / 64;            // loads per group
    constexpr int kPerChunk = 16 / kEsz;                 // elements per chunk
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int row = q * (64 / kChunks) + lane / kChunks;
        const int logical = (lane % kChunks) ^ (row & 15);
        int64_t tok = tok0 + row;
        tok = tok < rows ? tok : rows - 1;
        int64_t ch = b0 * 32 + logical * kPerChunk;
        ch = ch < cols ? ch : cols - kPerChunk;
        const uint8_t* src = static_cast<const uint8_t*>(x) + (tok * cols + ch) * kEsz;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + q * 1024), 16, 0, 0);
    }
}

template <bool kXBf16, bool kYBf16, bool kTiled>
__global__ __launch_bounds__(256) void block_transform_kernel(const void* __restrict__ x, int64_t rows,
                                                              int64_t cols, const uint16_t* __restrict__ t,
                                                              int64_t n_t, void* __restrict__ y,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
    constexpr int kEsz = kXBf16 ? 2 : 4;
    constexpr int kRowBytes = 128 * kEsz;                // 4 blocks of one token
    constexpr int kBufBytes = 32 * kRowBytes;            // one 32-token group (8 / 16 KiB)
    constexpr int kLoads = kBufBytes / 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t stage[4][2][kBufBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int h = lane >> 5;
    const int r32 = lane & 31;
    const int64_t nblk = cols / 32;
    const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * 4;   // first of this wave's 4 blocks
    if (b0 >= nblk) return;                                     // wave-uniform; no workgroup barriers below
    const int64_t tok_base = (int64_t)blockIdx.y * (32 * kTokIters);
    uint8_t* const bufs[2] = {stage[wave][0], stage[wave][1]};

    issue_group<kEsz>(bufs[0], x, rows, cols, tok_base, b0, lane);

    // A operand: lane holds T_b^T row r32 (= column r32 of T_b) at
    // k = 8h..8h+7 (first MFMA) and 16 + 8h.. (second MFMA).
    v8s tf[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t b = b0 + j < nblk ? b0 + j : nblk - 1;
        const uint16_t* tb = t + (n_t == 1 ? 0 : b) * 1024;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 8; ++e) tf[j][half][e] = (short)tb[(16 * half + 8 * h + e) * 32 + r32];
    }

#pragma unroll
    for (int it = 0; it < kTokIters; ++it) {
        const uint8_t* buf = bufs[it & 1];
        if (it + 1 < kTokIters) {
            // the other buffer was last read in iteration it - 1 (those reads
            // completed before their MFMAs): refill it with the next group
            issue_group<kEsz>(bufs[(it + 1) & 1], x, rows, cols, tok_base + (it + 1) * 32, b0, lane);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 7, 15));     // this group's loads landed
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 7, 15));
        }
        asm volatile("" ::: "memory");
        const int64_t tok = tok_base + it * 32 + r32;
        const bool live = tok < rows;
        const uint8_t* row = buf + r32 * kRowBytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t b = b0 + j;
            if (b >= nblk) break;                                   // wave-uniform
            // B operand: features 16 half + 8h .. +7 of block j for token r32.
            // A bf16 x is the operand itself.  An fp32 x is carried as three
            // bf16 parts hi + mid + lo (hi = bf16(x), mid = bf16(x - hi),
            // lo = bf16(x - hi - mid); the differences are exact in fp32),
            // which equal x exactly for |x| above about 2^-100, so y is
            // formed from the caller's values and only the order of the fp32
            // sums differs from x_b . T_b.
            v8s xf[2], xm[2], xl[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int g = 2 * half + h;                         // 8-feature group in the block
                if (kXBf16) {
                    const int c = (4 * j + g) ^ (r32 & 15);
                    const v4u v = *reinterpret_cast<const v4u*>(row + c * 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xf[half][2 * i] = (short)(v[i] & 0xFFFFu);
                        xf[half][2 * i + 1] = (short)(v[i] >> 16);
                    }
                } else {
                    const int c0 = (8 * j + 2 * g) ^ (r32 & 15), c1 = (8 * j + 2 * g + 1) ^ (r32 & 15);
                    const v4f v0 = *reinterpret_cast<const v4f*>(row + c0 * 16);
                    const v4f v1 = *reinterpret_cast<const v4f*>(row + c1 * 16);
                    const float xv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const uint32_t ph = pack_bf16x2(xv[e], xv[e + 1]);
                        const float ra = xv[e] - bf16_bits_to_f32(ph & 0xFFFFu);
                        const float rb = xv[e + 1] - bf16_bits_to_f32(ph >> 16);
                        const uint32_t pm = pack_bf16x2(ra, rb);
                        const uint32_t pl = pack_bf16x2(ra - bf16_bits_to_f32(pm & 0xFFFFu),
                                                        rb - bf16_bits_to_f32(pm >> 16));
                        xf[half][e] = (short)(ph & 0xFFFFu);
                        xf[half][e + 1] = (short)(ph >> 16);
                        xm[half][e] = (short)(pm & 0xFFFFu);
                        xm[half][e + 1] = (short)(pm >> 16);
                        xl[half][e] = (short)(pl & 0xFFFFu);
                        xl[half][e + 1] = (short)(pl >> 16);
                    }
                }
            }
            v16f acc = {};
            if (!kXBf16) {                                          // smallest parts first
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][0], xl[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][1], xl[1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][0], xm[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][1], xm[1], acc, 0, 0, 0);
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][0], xf[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[j][1], xf[1], acc, 0, 0, 0);
            float hv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) hv[i] = acc[i];
            if (y != nullptr && live) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int64_t o = tok * cols + b * 32 + 8 * a + 4 * h;
                    if (kYBf16) {
                        v2u v;
                        v[0] = pack_bf16x2(hv[4 * a], hv[4 * a + 1]);
                        v[1] = pack_bf16x2(hv[4 * a + 2], hv[4 * a + 3]);
                        *reinterpret_cast<v2u*>(static_cast<uint16_t*>(y) + o) = v;
                    } else {
                        *reinterpret_cast<v4f*>(static_cast<float*>(y) + o) =
                            (v4f){hv[4 * a], hv[4 * a + 1], hv[4 * a + 2], hv[4 * a + 3]};
                    }
                }
            }
            if (codes != nullptr) {
                if (kTiled)
                    store_mx_block(hv, lane, live, codes + tiled_code_off(tok, b * 32, cols),
                                   scales + tiled_scale_off(tok, b, cols));
                else
                    store_mx_block(hv, lane, live, codes + tok * (cols / 2) + b * 16, scales + tok * nblk + b);
            }
        }
    }
}

// W'_b = T_b^-1 . W_b.  One workgroup per (block b, 256 columns): the
// workgroup LU-factorises T_b in fp64 with partial pivoting in LDS, then every thread
// solves for one column (forward then back substitution) and stores fp32.
__global__ __launch_bounds__(256) void fold_inverse_kernel(const float* __restrict__ w, int64_t K, int64_t N,
                                                           const uint16_t* __restrict__ t, int64_t n_t,
                                                           float* __restrict__ w_out) {
    __shared__ double lu[32][33];
    __shared__ int perm[32];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const uint16_t* tb = t + (n_t == 1 ? 0 : b) * 1024;
    for (int i = tid; i < 1024; i += 256) lu[i / 32][i % 32] = (double)bf16_bits_to_f32(tb[i]);
    if (tid < 32) perm[tid] = tid;
    __syncthreads();
    for (int k = 0; k < 32; ++k) {
        // pivot: largest |lu[i][k]| over i >= k (first of equals), by thread 0
        if (tid == 0) {
            int p = k;
            double best = fabs(lu[k][k]);
            for (int i = k + 1; i < 32; ++i) {
                const double v = fabs(lu[i][k]);
                if (v > best) { best = v; p = i; }
            }
            if (p != k) {
                for (int j = 0; j < 32; ++j) {
                    const double tmp = lu[k][j]; lu[k][j] = lu[p][j]; lu[p][j] = tmp;
                }
                const int tp = perm[k]; perm[k] = perm[p]; perm[p] = tp;
            }
        }
        __syncthreads();
        if (tid > k && tid < 32) lu[tid][k] /= lu[k][k];
        __syncthreads();
        for (int e = tid; e < 32 * 32; e += 256) {
            const int i = e / 32, j = e % 32;
            if (i > k && j > k) lu[i][j] -= lu[i][k] * lu[k][j];
        }
        __syncthreads();
    }
    const int64_t n = (int64_t)blockIdx.x * 256 + tid;
    if (n >= N) return;
    double v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (double)w[(b * 32 + perm[i]) * N + n];
#pragma unroll
    for (int i = 1; i < 32; ++i)
#pragma unroll
        for (int j = 0; j < i; ++j) v[i] -= lu[i][j] * v[j];
#pragma unroll
    for (int i = 31; i >= 0; --i) {
#pragma unroll
        for (int j = i + 1; j < 32; ++j) v[i] -= lu[i][j] * v[j];
        v[i] /= lu[i][i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) w_out[(b * 32 + i) * N + n] = (float)v[i];
}

}  // namespace

hipError_t launch_block_transform(const void* x, bool x_bf16, int64_t rows, int64_t cols,
                                  const uint16_t* t, int64_t n_t, void* y, bool y_bf16,
                                  uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream) {
    const int64_t nblk = cols / 32;
    const int64_t wg_cols = (nblk + 15) / 16;                  // 4 waves x 4 blocks per workgroup
    const int64_t wg_rows = (rows + 32 * kTokIters - 1) / (32 * kTokIters);
    const dim3 grid((unsigned)wg_cols, (unsigned)wg_rows);
#define FP4DIT_LAUNCH_BT(XB, YB, T) \
    hipLaunchKernelGGL((block_transform_kernel<XB, YB, T>), grid, dim3(256), 0, stream, x, rows, cols, t, n_t, y, \
                       codes, scales)
#define FP4DIT_LAUNCH_BT2(XB, YB) \
    if (tiled) FP4DIT_LAUNCH_BT(XB, YB, true); else FP4DIT_LAUNCH_BT(XB, YB, false)
    if (x_bf16) {
        if (y_bf16) { FP4DIT_LAUNCH_BT2(true, true); } else { FP4DIT_LAUNCH_BT2(true, false); }
    } else {
        if (y_bf16) { FP4DIT_LAUNCH_BT2(false, true); } else { FP4DIT_LAUNCH_BT2(false, false); }
    }
#undef FP4DIT_LAUNCH_BT2
#undef FP4DIT_LAUNCH_BT
    return hipGetLastError();
}

hipError_t launch_fold_inverse(const float* w, int64_t K, int64_t N, const uint16_t* t, int64_t n_t,
                               float* w_out, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / 32));
    hipLaunchKernelGGL(fold_inverse_kernel, grid, dim3(256), 0, stream, w, K, N, t, n_t, w_out);
    return hipGetLastError();
}

}  // namespace fp4dit
