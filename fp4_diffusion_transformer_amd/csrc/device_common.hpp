// Device helpers shared by the fp4dit HIP kernels (gfx950 / CDNA4).
//
// MXFP4 encoding (fal, "Running the transformer in FP4": 1 sign, 2 exponent,
// 1 mantissa bit per element; KroQuant, "Deep analysis": MXFP4, one
// power-of-two scale per 32 elements).  The rules are fixed by the C ABI
// (include/fp4dit.h): shared exponent floor(log2 amax) - 2 clamped to
// [-127, 127]; round to nearest, ties to even mantissa; saturate at 6; sign
// copied.  The block scale is derived from the fp32 bit pattern with integer
// arithmetic (exact for subnormal inputs, independent of the denormal mode).
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
// Shared exponent of a block from the bits of its largest magnitude (sign
// bit clear).  Returns the e8m0 byte (shared + 127) of shared =
// clamp(floor(log2 amax) - 2, -127, 127): for a normal amax with exponent
// field e that is max(e - 2, 0) (e - 129 never exceeds 125); a subnormal
// amax has floor(log2) - 2 <= -129, clamped to byte 0, and so has zero --
// the same max(e - 2, 0) with e = 0.  Inf / NaN (e = 255): 0xFF.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 23;
    const uint32_t s = e > 2u ? e - 2u : 0u;
    return e >= 255u ? 0xFFu : s;
}

// Largest magnitude of n fp32 values, as sign-cleared bits (a NaN ranks
// above Inf, Inf above every finite value).  Two max chains over the raw
// bits instead of a mask per value: as signed integers the non-negative
// floats order by magnitude and beat every negative one; as unsigned
// integers the negative ones order by magnitude and beat every
// non-negative one.
template <int N>
__device__ __forceinline__ uint32_t amax_bits(const float* v) {
    int si = (int)__float_as_uint(v[0]);
    uint32_t su = __float_as_uint(v[0]);
#pragma unroll
    for (int i = 1; i < N; ++i) {
        const uint32_t b = __float_as_uint(v[i]);
        si = (int)b > si ? (int)b : si;
        su = b > su ? b : su;
    }
    const uint32_t a = (uint32_t)si & 0x7FFFFFFFu, c = su & 0x7FFFFFFFu;
    return a > c ? a : c;
}

// --------------------------------------------------------------- e2m1 -----
// Encode 8 fp32 values to 8 e2m1 codes packed in a uint32 (element i in
// nibble i, so element 2j sits in the low nibble of byte j) under the block
// scale byte sb, i.e. round(x / 2^(sb - 127)).
//
// Uses V_CVT_SCALEF32_PK_FP4_F32 (two values per instruction, into the byte
// picked by its select operand).  The fp32 scale operand is the e8m0 byte
// placed in an fp32 exponent field; the instruction takes its power of two
// (byte 0 gives 2^-127).  On the values a block can hold, |x| / 2^s < 8 with
// s the block's shared exponent, this conversion was checked bit for bit
// against a plain integer implementation of the encoding rule (nearest e2m1
// level, ties to even mantissa, saturation at 6, sign kept) for every finite
// bf16 value, millions of random fp32 values and every scale byte 0..254.
// A block with Inf / NaN (scale byte 0xFF) is not encoded: callers store 0.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* x, uint32_t scale_byte) {
    const float sc = __uint_as_float(scale_byte << 23);
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], sc, 3);
    return w;
}

// Encode 4 fp32 values to 4 codes in the low 16 bits (element i in nibble i).
__device__ __forceinline__ uint32_t e2m1_pack4(const float* x, uint32_t scale_byte) {
    const float sc = __uint_as_float(scale_byte << 23);
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], sc, 1);
    return w & 0xFFFFu;
}

// ------------------------------------------------------- tiled layout ----
// Byte offsets in the MX_TILED layout of a [rows][cols] MXFP4 matrix
// (cols % 128 == 0): codes in 128-byte tiles of 2 rows x 128 elements,
// scales in 128-byte tiles of 32 rows x 4 blocks (see include/fp4dit.h).
// tiled_code_off: byte holding elements (k, k+1) of row r, k even.
__device__ __forceinline__ int64_t tiled_code_off(int64_t r, int64_t k, int64_t cols) {
    return (((r >> 1) * (cols >> 7) + (k >> 7)) << 7) + ((r & 1) << 6) + ((k & 127) >> 1);
}
// tiled_scale_off: scale byte of row r, 32-element block b.
__device__ __forceinline__ int64_t tiled_scale_off(int64_t r, int64_t b, int64_t cols) {
    return (((r >> 5) * (cols >> 7) + (b >> 2)) << 7) + ((r & 31) << 2) + (b & 3);
}

// ---------------------------------------------------------------- bf16 ----
// fp32 -> bf16, round to nearest even, with V_CVT_PK_BF16_F32 (two values per
// instruction; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.0f) & 0xFFFFu;
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
