// Diffusion-sampler update kernels: ETD1, ETD2 and the Richardson combine.
//
// "拡散サンプリングの高速化：数値計算手法とスコアベースモデルの出会い"
// (Accelerating diffusion sampling: numerical methods meet score-based
// models), sections on the exponential integrator and on the fused update
// kernels: each update is a few elementwise operations, and one launch that
// reads every input once and writes the result once replaces a chain of
// intermediates:
//   ETD1        out = decay * x + coeff * x0
//   ETD2        out = decay * x + c0 * x0 + c1 * x0_prev
//   Richardson  out = (scale * fine - coarse) / (scale - 1)
// Storage fp32, bf16 or fp16 (the page's mixed precision: a 16-bit latent
// where the ODE is smooth), arithmetic fp32 with one rounding into the
// output type.  HBM-bound: every thread moves two 16-byte pieces per operand
// (4 fp32 or 8 16-bit elements each) with non-temporal accesses, laid out so
// that each load or store instruction covers 1 KiB of contiguous memory per
// wave.  (Two adjacent pieces per thread, i.e. half of each line per
// instruction, ran at 3.1 TB/s against 5.4 for this layout: a non-temporal
// access does not keep the line for the instruction that reads its other
// half.)  A ragged tail (n % piece) is taken element by element.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

enum SamplerOp { kEtd1 = 0, kEtd2 = 1, kRichardson = 2 };
enum Storage { kF32 = 0, kBf16 = 1, kF16 = 2 };

template <int S>
struct Elem;
template <>
struct Elem<kF32> {
    typedef float T;
    static __device__ __forceinline__ float get(T v) { return v; }
    static __device__ __forceinline__ T put(float f) { return f; }
};
template <>
struct Elem<kBf16> {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(T v) { return __uint_as_float((uint32_t)v << 16); }
    static __device__ __forceinline__ T put(float f) { return (T)f32_to_bf16_bits(f); }
};
template <>
struct Elem<kF16> {
    typedef _Float16 T;
    static __device__ __forceinline__ float get(T v) { return (float)v; }
    static __device__ __forceinline__ T put(float f) { return (T)f; }
};

// 8 elements of one operand: 16 bytes (16-bit types) or 32 bytes (fp32).
// One 16-byte piece: 16 / sizeof(T) elements.
template <int S>
struct Piece {
    static constexpr int kElems = 16 / (int)sizeof(typename Elem<S>::T);
};

template <int S>
__device__ __forceinline__ void load_piece(const typename Elem<S>::T* p, float* f) {
    typedef typename Elem<S>::T T;
    const v4u a = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    if (S == kF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(a[j]);
    } else {
        T e[8];
        __builtin_memcpy(e, &a, 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = Elem<S>::get(e[j]);
    }
}

template <int S>
__device__ __forceinline__ void store_piece(typename Elem<S>::T* p, const float* f) {
    typedef typename Elem<S>::T T;
    v4u a;
    if (S == kF32) {
        a = (v4u){__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    } else {
        T e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = Elem<S>::put(f[j]);
        __builtin_memcpy(&a, e, 16);
    }
    __builtin_nontemporal_store(a, reinterpret_cast<v4u*>(p));
}

template <int OP>
__device__ __forceinline__ float update(float a, float b, float c, float k0, float k1, float k2) {
    if (OP == kEtd1) return __builtin_fmaf(k1, b, k0 * a);
    if (OP == kEtd2) return __builtin_fmaf(k2, c, __builtin_fmaf(k1, b, k0 * a));
    return __builtin_fmaf(k0, a, -b) / k1;                 // k0 = scale, k1 = scale - 1
}

// a, b, c: x, x0, x0_prev (ETD) or fine, coarse (Richardson; c unused).
constexpr int kPieces = 2;                 // 16-byte pieces per thread per operand

template <int OP, int S>
__global__ __launch_bounds__(256) void sampler_kernel(const typename Elem<S>::T* __restrict__ a,
                                                      const typename Elem<S>::T* __restrict__ b,
                                                      const typename Elem<S>::T* __restrict__ c, int64_t n,
                                                      float k0, float k1, float k2,
                                                      typename Elem<S>::T* __restrict__ out) {
    constexpr int E = Piece<S>::kElems;
    int64_t i0[kPieces];
    float fa[kPieces][8], fb[kPieces][8], fc[kPieces][8];
    // piece (block * kPieces + j) * 256 + thread: instruction j of a wave
    // covers 64 consecutive pieces
#pragma unroll
    for (int j = 0; j < kPieces; ++j) i0[j] = (((int64_t)blockIdx.x * kPieces + j) * 256 + threadIdx.x) * E;
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
        if (i0[j] + E <= n) {
            load_piece<S>(a + i0[j], fa[j]);
            load_piece<S>(b + i0[j], fb[j]);
            if (OP == kEtd2) load_piece<S>(c + i0[j], fc[j]);
        }
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
        if (i0[j] + E <= n) {
            float r[8];
#pragma unroll
            for (int e = 0; e < E; ++e) r[e] = update<OP>(fa[j][e], fb[j][e], OP == kEtd2 ? fc[j][e] : 0.f, k0, k1, k2);
            store_piece<S>(out + i0[j], r);
        } else if (i0[j] < n) {                         // the ragged tail
            for (int64_t i = i0[j]; i < n; ++i) {
                const float x2 = OP == kEtd2 ? Elem<S>::get(c[i]) : 0.f;
                out[i] = Elem<S>::put(update<OP>(Elem<S>::get(a[i]), Elem<S>::get(b[i]), x2, k0, k1, k2));
            }
        }
    }
}

template <int OP>
hipError_t launch_op(const void* a, const void* b, const void* c, int64_t n, int storage, float k0, float k1,
                     float k2, void* out, hipStream_t stream) {
    const int64_t per_wg = 256 * kPieces * (storage == kF32 ? 4 : 8);
    const dim3 grid((unsigned)((n + per_wg - 1) / per_wg));
#define FP4DIT_S(S)                                                                                        \
    hipLaunchKernelGGL((sampler_kernel<OP, S>), grid, dim3(256), 0, stream,                                \
                       static_cast<const typename Elem<S>::T*>(a), static_cast<const typename Elem<S>::T*>(b), \
                       static_cast<const typename Elem<S>::T*>(c), n, k0, k1, k2,                          \
                       static_cast<typename Elem<S>::T*>(out))
    if (storage == kF32) FP4DIT_S(kF32);
    else if (storage == kBf16) FP4DIT_S(kBf16);
    else FP4DIT_S(kF16);
#undef FP4DIT_S
    return hipGetLastError();
}

}  // namespace

hipError_t launch_etd1(const void* x, const void* x0, int64_t n, int storage, float decay, float coeff, void* out,
                       hipStream_t stream) {
    return launch_op<kEtd1>(x, x0, nullptr, n, storage, decay, coeff, 0.f, out, stream);
}

hipError_t launch_etd2(const void* x, const void* x0, const void* x0_prev, int64_t n, int storage, float decay,
                       float c0, float c1, void* out, hipStream_t stream) {
    return launch_op<kEtd2>(x, x0, x0_prev, n, storage, decay, c0, c1, out, stream);
}

hipError_t launch_richardson(const void* fine, const void* coarse, int64_t n, int storage, float scale, void* out,
                             hipStream_t stream) {
    return launch_op<kRichardson>(fine, coarse, nullptr, n, storage, scale, scale - 1.0f, 0.f, out, stream);
}

}  // namespace fp4dit
