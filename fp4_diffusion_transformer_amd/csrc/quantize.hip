// MXFP4 quantisation kernels: online activation quantisation and offline
// weight packing (transpose to [N][K], optional SwiGLU column interleave).
//
// fal, "Running the transformer in FP4" (e2m1 elements) and the QAD section
// (weights quantised statically for inference); KroQuant, "Deep analysis"
// (MXFP4: 32-element blocks with a shared power-of-two scale); fal, "Fusing
// gated SiLU" (gate/up columns permuted once at packing time).
//
// Activation quantisation is HBM-bound: 2 (bf16) or 4 (fp32) bytes in and
// 17/32 byte out per element.  Four lanes share a 32-element block; each
// lane takes 8 consecutive elements (16 B of bf16), so a wave reads 1 KiB of
// contiguous memory per load; the input is read once (non-temporal loads for
// bf16, whose 16-byte pieces cover whole lines per wave).
// The block amax is reduced over the four lanes with DPP quad permutes.
// Measured on 4096 x 4096 bf16: one 8-element unit per thread (many small
// workgroups) beats 2, 4 or 8 units per thread with all loads issued first,
// and plain 4-byte code stores per lane beat gathering a block's codes (and
// four blocks' scales) into one lane with DPP for a single wider store.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {

constexpr int kQuantUnits = 1;                   // 8-element units per thread

template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t nunits, int64_t cols) {
    uint32_t xb[kQuantUnits][8];
    int64_t unit[kQuantUnits];
#pragma unroll
    for (int i = 0; i < kQuantUnits; ++i) {
        unit[i] = ((int64_t)blockIdx.x * kQuantUnits + i) * 256 + threadIdx.x;
        if (unit[i] >= nunits) continue;         // whole quads leave together (nunits % 4 == 0)
        const int64_t elem = unit[i] * 8;
        if (kBf16) {
            const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(static_cast<const uint16_t*>(x) + elem));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xb[i][2 * j] = v[j] << 16;
                xb[i][2 * j + 1] = v[j] & 0xFFFF0000u;
            }
        } else {
            // fp32: a lane's 8 elements are two adjacent 16-byte pieces, so
            // each load covers half of every line it touches; ordinary
            // (cached) loads let the second one hit the line the first
            // brought in (non-temporal ones fetched it twice)
            const v4u* p = reinterpret_cast<const v4u*>(static_cast<const float*>(x) + elem);
            const v4u v0 = p[0], v1 = p[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xb[i][j] = v0[j];
                xb[i][4 + j] = v1[j];
            }
        }
    }
    const int part = (int)(threadIdx.x & 3);
#pragma unroll
    for (int i = 0; i < kQuantUnits; ++i) {
        if (unit[i] >= nunits) continue;
        const int64_t blk = unit[i] >> 2;
        uint32_t amax = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t a = xb[i][j] & 0x7FFFFFFFu;
            amax = a > amax ? a : amax;
        }
        amax = max_quad_u(amax);
        const uint32_t sc = e8m0_from_amax_bits(amax);
        float xf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xf[j] = __uint_as_float(xb[i][j]);
        const uint32_t enc = e2m1_pack8(xf, sc);
        const uint32_t w = sc == 0xFFu ? 0u : enc;   // Inf / NaN block: zero codes
        if (kTiled) {
            const uint32_t nbr = (uint32_t)(cols >> 5);              // blocks per row (nblocks < 2^32)
            const uint32_t row = (uint32_t)blk / nbr, b = (uint32_t)blk - row * nbr;
            *reinterpret_cast<uint32_t*>(codes + tiled_code_off(row, (int64_t)b * 32 + part * 8, cols)) = w;
            if (part == 0) scales[tiled_scale_off(row, b, cols)] = (uint8_t)sc;
        } else {
            reinterpret_cast<uint32_t*>(codes)[unit[i]] = w;
            if (part == 0) scales[blk] = (uint8_t)sc;
        }
    }
}

// QAD fake quantisation (fal, QAD section: the forward pass goes through the
// FP4 rounding, the backward pass passes the gradient straight through, so
// it needs no kernel): y = D(Q(x)), blocks of 32 along the row, the same
// unit layout and encoding as quantize_kernel, then each code decoded back.
// The decoded values (e2m1 level times a power of two, at most two
// significant bits) are exact in fp32 and in bf16, including the subnormal
// ones (fp32 denormals are kept), so the bf16 result is the fp32 one with its
// low 16 bits, which are zero, dropped.  A block holding Inf / NaN gives NaN.
template <bool kBf16In, bool kBf16Out>
__global__ __launch_bounds__(256) void fake_quant_kernel(const void* __restrict__ x, void* __restrict__ y,
                                                         int64_t nunits) {
    const int64_t unit = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (unit >= nunits) return;                  // whole quads leave together (nunits % 4 == 0)
    const int64_t elem = unit * 8;
    uint32_t xb[8];
    if (kBf16In) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(static_cast<const uint16_t*>(x) + elem));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xb[2 * j] = v[j] << 16;
            xb[2 * j + 1] = v[j] & 0xFFFF0000u;
        }
    } else {
        const v4u* p = reinterpret_cast<const v4u*>(static_cast<const float*>(x) + elem);
        const v4u v0 = p[0], v1 = p[1];                 // cached: see quantize_kernel
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xb[j] = v0[j];
            xb[4 + j] = v1[j];
        }
    }
    uint32_t amax = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t a = xb[j] & 0x7FFFFFFFu;
        amax = a > amax ? a : amax;
    }
    const uint32_t sc = e8m0_from_amax_bits(max_quad_u(amax));
    float xf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = __uint_as_float(xb[j]);
    const uint32_t enc = e2m1_pack8(xf, sc);
    // level * 2 of magnitude codes 0..7 (0, 1, 2, 3, 4, 6, 8, 12), one nibble each
    constexpr uint32_t kTwiceLevel = 0xC8643210u;
    // 2^(shared - 1) = 2^(sc - 128): a normal fp32 for sc >= 2, else 2^-127 / 2^-128
    const uint32_t p2 = sc >= 2u ? (sc - 1u) << 23 : 0x00400000u >> (1u - sc);
    const float half_scale = __uint_as_float(p2);
    uint32_t yb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t c = (enc >> (4 * j)) & 15u;
        const float mag = (float)((kTwiceLevel >> (4 * (c & 7u))) & 15u) * half_scale;
        yb[j] = sc == 0xFFu ? 0x7FC00000u : (__float_as_uint(mag) | ((c & 8u) << 28));
    }
    if (kBf16Out) {
        v4u v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (yb[2 * j] >> 16) | (yb[2 * j + 1] & 0xFFFF0000u);
        __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(static_cast<uint16_t*>(y) + elem));
    } else {
        v4u* p = reinterpret_cast<v4u*>(static_cast<float*>(y) + elem);   // cached, as the loads
        p[0] = (v4u){yb[0], yb[1], yb[2], yb[3]};
        p[1] = (v4u){yb[4], yb[5], yb[6], yb[7]};
    }
}

// One thread per output block (physical column p, K-block kb): gathers the 32
// weights of logical column src(p), rows 32kb..32kb+31, and encodes them.
template <bool kBf16, bool kTiled>
__global__ __launch_bounds__(256) void pack_weight_kernel(const void* __restrict__ w,
                                                          int64_t K, int64_t N, int group,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t kb = blockIdx.y;
    if (p >= N) return;
    int64_t src = p;
    if (group > 0) {
        const int64_t j = (p / (2 * group)) * group + p % group;
        src = ((p / group) & 1) ? (N / 2 + j) : j;
    }
    uint32_t xb[32];
    uint32_t amax = 0u;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const int64_t idx = (kb * 32 + r) * N + src;
        uint32_t b;
        if (kBf16) {
            b = (uint32_t)static_cast<const uint16_t*>(w)[idx] << 16;
        } else {
            b = __float_as_uint(static_cast<const float*>(w)[idx]);
        }
        xb[r] = b;
        const uint32_t a = b & 0x7FFFFFFFu;
        amax = a > amax ? a : amax;
    }
    const uint32_t sc = e8m0_from_amax_bits(amax);
    float xf[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) xf[r] = __uint_as_float(xb[r]);
    v4u out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = sc == 0xFFu ? 0u : e2m1_pack8(xf + 8 * i, sc);
    if (kTiled) {
        *reinterpret_cast<v4u*>(codes + tiled_code_off(p, kb * 32, K)) = out;
        scales[tiled_scale_off(p, kb, K)] = (uint8_t)sc;
    } else {
        *reinterpret_cast<v4u*>(codes + p * (K / 2) + kb * 16) = out;
        scales[p * (K / 32) + kb] = (uint8_t)sc;
    }
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream) {
    const int64_t nunits = rows * (cols / 32) * 4;
    const int64_t per_wg = 256 * kQuantUnits;
    const dim3 grid((unsigned)((nunits + per_wg - 1) / per_wg));
#define FP4DIT_Q(B, T) \
    hipLaunchKernelGGL((quantize_kernel<B, T>), grid, dim3(256), 0, stream, x, codes, scales, nunits, cols)
    if (bf16) {
        if (tiled) FP4DIT_Q(true, true); else FP4DIT_Q(true, false);
    } else {
        if (tiled) FP4DIT_Q(false, true); else FP4DIT_Q(false, false);
    }
#undef FP4DIT_Q
    return hipGetLastError();
}

hipError_t launch_pack_weight(const void* w, bool bf16, int64_t K, int64_t N, int group,
                              uint8_t* codes, uint8_t* scales, bool tiled, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / 32));
#define FP4DIT_P(B, T) \
    hipLaunchKernelGGL((pack_weight_kernel<B, T>), grid, dim3(256), 0, stream, w, K, N, group, codes, scales)
    if (bf16) {
        if (tiled) FP4DIT_P(true, true); else FP4DIT_P(true, false);
    } else {
        if (tiled) FP4DIT_P(false, true); else FP4DIT_P(false, false);
    }
#undef FP4DIT_P
    return hipGetLastError();
}

hipError_t launch_fake_quant(const void* x, bool x_bf16, int64_t rows, int64_t cols, void* y, bool y_bf16,
                             hipStream_t stream) {
    const int64_t nunits = rows * (cols / 8);
    const dim3 grid((unsigned)((nunits + 255) / 256));
#define FP4DIT_FQ(A, B) hipLaunchKernelGGL((fake_quant_kernel<A, B>), grid, dim3(256), 0, stream, x, y, nunits)
    if (x_bf16) {
        if (y_bf16) FP4DIT_FQ(true, true); else FP4DIT_FQ(true, false);
    } else {
        if (y_bf16) FP4DIT_FQ(false, true); else FP4DIT_FQ(false, false);
    }
#undef FP4DIT_FQ
    return hipGetLastError();
}

}  // namespace fp4dit
