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
// output type.  HBM-bound: every thread moves 8 elements per operand with
// non-temporal 16-byte accesses; a ragged tail (n % 8) is taken element by
// element by the last thread.
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
template <int S>
__device__ __forceinline__ void load8(const typename Elem<S>::T* p, float* f) {
    typedef typename Elem<S>::T T;
    if (S == kF32) {
        const v4u a = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
        const v4u b = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[j] = __uint_as_float(a[j]);
            f[4 + j] = __uint_as_float(b[j]);
        }
    } else {
        const v4u a = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
        T e[8];
        __builtin_memcpy(e, &a, 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = Elem<S>::get(e[j]);
    }
}

template <int S>
__device__ __forceinline__ void store8(typename Elem<S>::T* p, const float* f) {
    typedef typename Elem<S>::T T;
    if (S == kF32) {
        __builtin_nontemporal_store((v4u){__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                                          __float_as_uint(f[3])}, reinterpret_cast<v4u*>(p));
        __builtin_nontemporal_store((v4u){__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                                          __float_as_uint(f[7])}, reinterpret_cast<v4u*>(p) + 1);
    } else {
        T e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = Elem<S>::put(f[j]);
        v4u a;
        __builtin_memcpy(&a, e, 16);
        __builtin_nontemporal_store(a, reinterpret_cast<v4u*>(p));
    }
}

template <int OP>
__device__ __forceinline__ float update(float a, float b, float c, float k0, float k1, float k2) {
    if (OP == kEtd1) return __builtin_fmaf(k1, b, k0 * a);
    if (OP == kEtd2) return __builtin_fmaf(k2, c, __builtin_fmaf(k1, b, k0 * a));
    return __builtin_fmaf(k0, a, -b) / k1;                 // k0 = scale, k1 = scale - 1
}

// a, b, c: x, x0, x0_prev (ETD) or fine, coarse (Richardson; c unused).
template <int OP, int S>
__global__ __launch_bounds__(256) void sampler_kernel(const typename Elem<S>::T* __restrict__ a,
                                                      const typename Elem<S>::T* __restrict__ b,
                                                      const typename Elem<S>::T* __restrict__ c, int64_t n,
                                                      float k0, float k1, float k2,
                                                      typename Elem<S>::T* __restrict__ out) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 + 8 <= n) {
        float fa[8], fb[8], fc[8], r[8];
        load8<S>(a + i0, fa);
        load8<S>(b + i0, fb);
        if (OP == kEtd2) load8<S>(c + i0, fc);
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = update<OP>(fa[j], fb[j], OP == kEtd2 ? fc[j] : 0.f, k0, k1, k2);
        store8<S>(out + i0, r);
    } else if (i0 < n) {                                    // the ragged tail
        for (int64_t i = i0; i < n; ++i) {
            const float fc = OP == kEtd2 ? Elem<S>::get(c[i]) : 0.f;
            out[i] = Elem<S>::put(update<OP>(Elem<S>::get(a[i]), Elem<S>::get(b[i]), fc, k0, k1, k2));
        }
    }
}

template <int OP>
hipError_t launch_op(const void* a, const void* b, const void* c, int64_t n, int storage, float k0, float k1,
                     float k2, void* out, hipStream_t stream) {
    const dim3 grid((unsigned)((n + 8 * 256 - 1) / (8 * 256)));
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
