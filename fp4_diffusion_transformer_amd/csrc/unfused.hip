// Stand-alone epilogue kernels: the unfused form of the per-head RMSNorm and
// SwiGLU epilogues, run on a bf16 GEMM output that has made the HBM round
// trip.
//
// fal, "Epilogue fusion in brief": without fusion the GEMM output goes to
// HBM and is read back by a second launch for each small op.  These kernels
// are that second launch, kept to measure on MI355X what the fused epilogue
// saves; they compute the same definitions (per-head RMSNorm with eps inside
// the square root and per-column gains; SiLU(gate) * up over the interleaved
// gate/up columns), on the bf16 values.
//
// Both are HBM-bound with no reuse: every thread moves 16-byte chunks (8
// bf16) with non-temporal loads and computes in fp32.
//  * RMSNorm: a head of hd columns is hd/8 consecutive lanes of one wave;
//    its sum of squares is reduced over those lanes with xor shuffles.
//  * SwiGLU: a thread reads the 8 gate and the 8 matching up values of 8
//    outputs (two chunks g columns apart) and writes one chunk.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

__device__ __forceinline__ void unpack8(const v4u v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(v[j] << 16);
        f[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ v4u pack8(const float* f) {
    v4u v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
    return v;
}

// One thread per 8-column chunk, chunks numbered row-major over the tensor
// (rows * cols / 8 < 2^32, checked by the host).
template <int kHd>
__global__ __launch_bounds__(256) void rmsnorm_head_kernel(const uint16_t* __restrict__ x, uint32_t n_chunks,
                                                           uint32_t row_chunks, int64_t n_norm,
                                                           const float* __restrict__ w, float eps,
                                                           uint16_t* __restrict__ y) {
    constexpr int kLanes = kHd / 8;                       // lanes per head: 16 or 32
    const uint32_t chunk = blockIdx.x * 256u + threadIdx.x;
    // every lane of a head takes part in the shuffles: cols % kHd == 0 keeps
    // a head's kLanes chunks consecutive and aligned, so whole heads are in
    // or out of range
    if (chunk >= n_chunks) return;
    const uint32_t row = chunk / row_chunks;
    const int64_t col = (int64_t)(chunk - row * row_chunks) * 8;
    const int64_t off = (int64_t)chunk * 8;
    float v[8];
    unpack8(__builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + off)), v);
    if (col < n_norm) {                                   // n_norm % kHd == 0: uniform per head
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
#pragma unroll
        for (int m = 1; m < kLanes; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float rstd = rsqrtf(ss * (1.0f / kHd) + eps);
        const v4f w0 = *reinterpret_cast<const v4f*>(w + col), w1 = *reinterpret_cast<const v4f*>(w + col + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = v[j] * rstd * w0[j];
            v[4 + j] = v[4 + j] * rstd * w1[j];
        }
    }
    __builtin_nontemporal_store(pack8(v), reinterpret_cast<v4u*>(y + off));
}

// One thread per 8 outputs, chunks numbered row-major over the output
// (rows * n_phys / 16 < 2^32).  Physical column p of the interleaved input is
// gate (p / g even) or up (p / g odd) of output (p / 2g) * g + p % g.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ c, uint32_t n_chunks,
                                                     uint32_t row_chunks, int group, uint16_t* __restrict__ h) {
    const uint32_t chunk = blockIdx.x * 256u + threadIdx.x;
    if (chunk >= n_chunks) return;
    const uint32_t row = chunk / row_chunks;
    const uint32_t o = (chunk - row * row_chunks) * 8;    // first output of the chunk in its row
    const uint32_t pg = (o / group) * 2 * group + o % group;   // its gate column (g % 8 == 0)
    const uint16_t* src = c + (int64_t)row * row_chunks * 16 + pg;
    float gt[8], up[8], r[8];
    // cached loads: the gate and up loads each cover every other 64-byte
    // half of the lines they touch (non-temporal loads fetched each line twice)
    unpack8(*reinterpret_cast<const v4u*>(src), gt);
    unpack8(*reinterpret_cast<const v4u*>(src + group), up);
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = gt[j] * __builtin_amdgcn_rcpf(1.0f + __expf(-gt[j])) * up[j];
    __builtin_nontemporal_store(pack8(r), reinterpret_cast<v4u*>(h + (int64_t)chunk * 8));
}

}  // namespace

hipError_t launch_rmsnorm_head(const uint16_t* x, int64_t rows, int64_t cols, int head_dim, int64_t n_norm,
                               const float* w, float eps, uint16_t* y, hipStream_t stream) {
    const uint32_t row_chunks = (uint32_t)(cols / 8), n_chunks = (uint32_t)(rows * (cols / 8));
    const dim3 grid((n_chunks + 255u) / 256u);
    if (head_dim == 128)
        hipLaunchKernelGGL(rmsnorm_head_kernel<128>, grid, dim3(256), 0, stream, x, n_chunks, row_chunks, n_norm, w,
                           eps, y);
    else
        hipLaunchKernelGGL(rmsnorm_head_kernel<256>, grid, dim3(256), 0, stream, x, n_chunks, row_chunks, n_norm, w,
                           eps, y);
    return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* c, int64_t rows, int64_t n_phys, int group, uint16_t* h,
                         hipStream_t stream) {
    const uint32_t row_chunks = (uint32_t)(n_phys / 16), n_chunks = (uint32_t)(rows * (n_phys / 16));
    const dim3 grid((n_chunks + 255u) / 256u);
    hipLaunchKernelGGL(swiglu_kernel, grid, dim3(256), 0, stream, c, n_chunks, row_chunks, group, h);
    return hipGetLastError();
}

}  // namespace fp4dit
