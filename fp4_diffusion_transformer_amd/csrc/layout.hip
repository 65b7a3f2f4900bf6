// Re-layout of an MXFP4 tensor between the row-major layout and the tiled
// layout the GEMM reads (both defined in include/fp4dit.h).  The codes and
// scale bytes move; no value changes.
//
// MXFP4 itself (KroQuant, "Deep analysis"; fal, "Running the transformer in
// FP4"): 4-bit e2m1 elements, two per byte, and one e8m0 scale byte per 32
// consecutive elements of a row.
//
// HBM-bound byte permutation, off the hot path (weight or interchange
// preparation).  One thread per 16-byte unit of output codes (16 bytes are
// contiguous in both layouts: a tiled row segment is 64 bytes), then one per
// output scale byte; grid-stride loop.  Padding rows of a tiled output are
// written as zero.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

// Byte offset of (row r, byte b of the row's cols/2 code bytes).
__device__ __forceinline__ int64_t code_byte(bool tiled, int64_t r, int64_t b, int64_t half, int64_t kq) {
    return tiled ? (((r >> 1) * kq + (b >> 6)) << 7) + ((r & 1) << 6) + (b & 63) : r * half + b;
}

// Byte offset of the scale of (row r, 32-element block blk).
__device__ __forceinline__ int64_t scale_byte(bool tiled, int64_t r, int64_t blk, int64_t nblk, int64_t kq) {
    return tiled ? (((r >> 5) * kq + (blk >> 2)) << 7) + ((r & 31) << 2) + (blk & 3) : r * nblk + blk;
}

template <bool kInTiled, bool kOutTiled>
__global__ __launch_bounds__(256) void relayout_kernel(const uint8_t* __restrict__ in_codes,
                                                       const uint8_t* __restrict__ in_scales, int64_t rows,
                                                       int64_t cols, uint8_t* __restrict__ out_codes,
                                                       uint8_t* __restrict__ out_scales, int64_t code_units,
                                                       int64_t scale_bytes) {
    const int64_t half = cols / 2, nblk = cols / 32, kq = cols / 128;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < code_units + scale_bytes; u += stride) {
        if (u < code_units) {
            const int64_t o = u * 16;
            int64_t r, b;
            if (kOutTiled) {
                const int64_t tile = o >> 7, within = o & 127;
                r = (tile / kq) * 2 + (within >> 6);
                b = (tile % kq) * 64 + (within & 63);
            } else {
                r = o / half;
                b = o % half;
            }
            v4u v = {0u, 0u, 0u, 0u};
            if (r < rows) v = *reinterpret_cast<const v4u*>(in_codes + code_byte(kInTiled, r, b, half, kq));
            *reinterpret_cast<v4u*>(out_codes + o) = v;
        } else {
            const int64_t o = u - code_units;
            int64_t r, blk;
            if (kOutTiled) {
                const int64_t tile = o >> 7, within = o & 127;
                r = (tile / kq) * 32 + (within >> 2);
                blk = (tile % kq) * 4 + (within & 3);
            } else {
                r = o / nblk;
                blk = o % nblk;
            }
            out_scales[o] = r < rows ? in_scales[scale_byte(kInTiled, r, blk, nblk, kq)] : (uint8_t)0;
        }
    }
}

}  // namespace

hipError_t launch_relayout(const uint8_t* in_codes, const uint8_t* in_scales, bool in_tiled, int64_t rows,
                           int64_t cols, uint8_t* out_codes, uint8_t* out_scales, bool out_tiled,
                           hipStream_t stream) {
    const int64_t code_rows = out_tiled ? (rows + 1) / 2 * 2 : rows;
    const int64_t scale_rows = out_tiled ? (rows + 31) / 32 * 32 : rows;
    const int64_t code_units = code_rows * (cols / 2) / 16;
    const int64_t scale_bytes = scale_rows * (cols / 32);
    const int64_t total = code_units + scale_bytes;
    const int64_t wgs = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
    const dim3 grid((unsigned)wgs);
#define FP4DIT_LAUNCH_RL(I, O)                                                                              \
    hipLaunchKernelGGL((relayout_kernel<I, O>), grid, dim3(256), 0, stream, in_codes, in_scales, rows, cols, \
                       out_codes, out_scales, code_units, scale_bytes)
    if (in_tiled) {
        if (out_tiled) FP4DIT_LAUNCH_RL(true, true); else FP4DIT_LAUNCH_RL(true, false);
    } else {
        if (out_tiled) FP4DIT_LAUNCH_RL(false, true); else FP4DIT_LAUNCH_RL(false, false);
    }
#undef FP4DIT_LAUNCH_RL
    return hipGetLastError();
}

}  // namespace fp4dit
