// Shader-clock probe (libfp4dit_clock.so), a measurement helper and no step
// of the method, built apart from libfp4dit.so.
//
// The MXFP4 roofline is quoted at the published 2.4 GHz, but under a
// sustained FP4 MFMA load the shader clock settles lower (power).  Each wave
// of the probe runs `iters` rounds of 16 independent scaled FP4 MFMAs
// (32x32x64, pseudo-random operands: the clock depends on the data) and
// records, around them, the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime); their ratio times 100 MHz is
// the clock that wave ran at.  One workgroup per CU loads the whole chip
// the way the persistent GEMM does; a single workgroup reads the clock of a
// lightly loaded chip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4dit_clock.h"

namespace {

typedef int v8i_ __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {        // an integer hash (operand bits)
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    return x ^ (x >> 16);
}

__global__ __launch_bounds__(256, 1) void clock_probe_kernel(uint64_t* __restrict__ out, int iters) {
    // the wave index in a scalar register and the lane recounted at the end,
    // so no per-lane id stays live across the MFMA loop
    const uint32_t wave_id = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t seed = (wave_id * 64u + (threadIdx.x & 63u)) * 64u;
    v8i_ a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[i][j] = j < 4 ? (int)mix32(seed + i * 8 + j) : 0;          // the FP4 MFMA reads 4 registers
            b[i][j] = j < 4 ? (int)mix32(seed + 32 + i * 8 + j) : 0;
        }
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, 127, 0,
                                                                           127);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    if (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0) {   // lane 0: vector stores
        out[3 * wave_id] = t1 - t0;
        out[3 * wave_id + 1] = r1 - r0;
        out[3 * wave_id + 2] = __float_as_uint(s);   // keeps the MFMAs
    }
}

}  // namespace

extern "C" int32_t fp4dit_clock_probe(uint64_t* out, int32_t workgroups, int32_t iters, hipStream_t stream) {
    if (!out) return 1;
    if (reinterpret_cast<uintptr_t>(out) % 8 != 0) return 3;
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20)) return 2;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(256), 0, stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
