// Device helpers shared by the fp4dit HIP kernels (gfx950 / CDNA4).
//
// MXFP4 encoding (fal, "Running the transformer in FP4": 1 sign, 2 exponent,
// 1 mantissa bit per element; KroQuant, "Deep analysis": MXFP4, one
// power-of-two scale per 32 elements).  The rules are fixed by the C ABI
// (include/fp4dit.h): shared exponent floor(log2 amax) - 2 clamped to
// [-127, 127]; round to nearest, ties to even mantissa; saturate at 6; sign
// copied.  Everything below works on the fp32 bit pattern with integer
// arithmetic, so it is exact for subnormal inputs and independent of the
// FP denormal mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dit {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- e8m0 ----
// Shared exponent of a block from the bits of its largest magnitude.
// Returns the e8m0 byte (shared + 127); 0xFF when amax is Inf or NaN.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
    if (amax_bits >= 0x7F800000u) return 0xFFu;          // Inf / NaN: unsupported
    if (amax_bits == 0u) return 0u;                      // all-zero block
    const uint32_t e = amax_bits >> 23;
    int floor_log2;
    if (e != 0u) {
        floor_log2 = (int)e - 127;
    } else {                                             // subnormal amax
        floor_log2 = (31 - __builtin_clz(amax_bits)) - 149;
    }
    int shared = floor_log2 - 2;
    shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
    return (uint32_t)(shared + 127);
}

// --------------------------------------------------------------- e2m1 -----
// 4-bit code of one fp32 value (bits) under shared exponent s = byte - 127.
// |q| = |x| / 2^s lies in [0, 8).  The grid step is 2^t with t = -1 below 2,
// 0 in [2, 4) and 1 from 4; n = RNE(|q| / 2^t) and the magnitude code is
// min(n + 2(t + 1), 7), which also saturates 8 to 6.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t xbits, uint32_t scale_byte) {
    const uint32_t sign = (xbits >> 28) & 8u;
    const uint32_t a = xbits & 0x7FFFFFFFu;
    const int s = (int)scale_byte - 127;
    // thresholds 2^(s+1) and 2^(s+2) as fp32 bit patterns (s + 129 <= 254 for finite data)
    const uint32_t two_bits = (uint32_t)(s + 128) << 23;
    const uint32_t four_bits = (uint32_t)(s + 129) << 23;
    const int t = a >= four_bits ? 1 : (a >= two_bits ? 0 : -1);
    const uint32_t e = a >> 23;
    const uint32_t sig = (a & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    const int e0 = e ? (int)e - 150 : -149;              // |x| = sig * 2^e0
    const int sh = s + t - e0;                           // n = RNE(sig >> sh)
    uint32_t n;
    if (sh >= 26) {
        n = 0u;                                          // |q| / 2^t < 1/4: rounds to 0
    } else {
        const uint32_t q = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u);
        const uint32_t half = 1u << (sh - 1);
        n = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
    }
    uint32_t mag = n + (uint32_t)(2 * (t + 1));
    mag = mag > 7u ? 7u : mag;
    return sign | mag;
}

// Encode 8 fp32 values (bits) to 8 codes packed in a uint32, element i in
// nibble i (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t e2m1_pack8(const uint32_t* xb, uint32_t scale_byte) {
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(xb[i], scale_byte) << (4 * i);
    return w;
}

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u | ((u >> 16) & 0x8000u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// ------------------------------------------------------- lane exchanges ----
// x[l] + x[l ^ 32] on every lane, with one v_permlane32_swap.
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t max_xor32_u(uint32_t x) {
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] > r[1] ? r[0] : r[1];
}

// Value held by lane l ^ 32.
__device__ __forceinline__ uint32_t partner_xor32(uint32_t x, int lane) {
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return lane < 32 ? r[1] : r[0];
}

// Max over each aligned group of 4 lanes (DPP quad permutes, no LDS).
__device__ __forceinline__ uint32_t max_quad_u(uint32_t x) {
    uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // lane ^ 1
    x = x > y ? x : y;
    y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);           // lane ^ 2
    return x > y ? x : y;
}

}  // namespace fp4dit
