// Load plan of the fused GEMM: the per-lane byte offsets of its direct-to-LDS
// operand loads into the MX_TILED operand buffers, and which K stage each
// load fetches.  Plain integer arithmetic, compiled for the device (the GEMM
// kernel) and for the host (a CPU test walks every load of a launch against
// the buffer sizes; the buffer loads' scalar stage offset is not covered by
// the hardware's range check, so every load must be in bounds by itself).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dit {
namespace plan {

constexpr int kBK = 128;    // K elements per stage: 64 code bytes and 4 scale bytes per row

// Operands are MX_TILED: K stage kt of rows (2p, 2p+1) is one 128-byte code
// tile at ((p * K/128) + kt) * 128, and stage kt of 32 rows is one 128-byte
// scale tile, so every load fetches whole cache lines.  kq = K / 128.
__host__ __device__ __forceinline__ uint32_t code_tile_off(uint32_t r, uint32_t kq) {
    return ((r >> 1) * kq) * 128 + (r & 1) * 64;
}
__host__ __device__ __forceinline__ uint32_t scale_tile_off(uint32_t r, uint32_t kq) {
    return ((r >> 5) * kq) * 128 + (r & 31) * 4;
}

// Bytes the kernel's buffer descriptors cover (the tiled buffers' sizes:
// codes padded to an even number of rows, scales to a multiple of 32).
__host__ __device__ __forceinline__ int64_t code_bytes(int64_t rows, int64_t K) { return ((rows + 1) & ~int64_t(1)) * (K / 2); }
__host__ __device__ __forceinline__ int64_t scale_bytes(int64_t rows, int64_t K) { return ((rows + 31) & ~int64_t(31)) * (K / 32); }

// Full 256 x 256 tile: each wave loads 64 of the 256 weight rows and 64 of
// the 256 token rows; one instruction moves 16 rows x 64 B (lane: row
// lane/4, 16-byte chunk lane%4, written at its swizzled LDS position), the
// scale instructions 64 rows x 4 B.  Token rows past M are clamped to row
// M - 1 (loaded, never stored).  A K stage adds its offset (stage * 128,
// see stage_soff) to every offset.
struct LoadPlan {
    uint32_t w_code[4], x_code[4];
    uint32_t w_scale, x_scale;
};

__host__ __device__ __forceinline__ LoadPlan make_plan(int M, int K, int n0, int m0, int wave, int lane) {
    LoadPlan p;
    const uint32_t kq = (uint32_t)(K / kBK);            // K stages (tiles per row pair / row block)
    const int rin = lane >> 2;                          // row within a 16-row group
    const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);  // chunk for physical slot lane & 3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (wave * 4 + j) * 16 + rin;
        p.w_code[j] = code_tile_off((uint32_t)(n0 + row), kq) + lchunk * 16;
        const int xr = m0 + row < M ? m0 + row : M - 1;
        p.x_code[j] = code_tile_off((uint32_t)xr, kq) + lchunk * 16;
    }
    p.w_scale = scale_tile_off((uint32_t)(n0 + wave * 64 + lane), kq);
    const int xr = m0 + wave * 64 + lane < M ? m0 + wave * 64 + lane : M - 1;
    p.x_scale = scale_tile_off((uint32_t)xr, kq);
    return p;
}

// Quarter tile (256 channels x 64 tokens): per stage a wave loads 4 weight
// code chunks of 16 rows (as in the full tile), 16 token rows, its 64 weight
// scale rows and all 64 token scale rows (every wave writes the same bytes
// to the same LDS place: one unconditional load, no lane mask).
struct QPlan {
    uint32_t w_code[4], x_code, w_scale, x_scale;
};

__host__ __device__ __forceinline__ QPlan make_qplan(int M, int K, int n0, int m0, int wave, int lane) {
    QPlan p;
    const uint32_t kq = (uint32_t)(K / kBK);
    const int rin = lane >> 2;
    const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        p.w_code[j] = code_tile_off((uint32_t)(n0 + (wave * 4 + j) * 16 + rin), kq) + lchunk * 16;
    const int xr = m0 + wave * 16 + rin < M ? m0 + wave * 16 + rin : M - 1;
    p.x_code = code_tile_off((uint32_t)xr, kq) + lchunk * 16;
    p.w_scale = scale_tile_off((uint32_t)(n0 + wave * 64 + lane), kq);
    const int sr = m0 + lane < M ? m0 + lane : M - 1;
    p.x_scale = scale_tile_off((uint32_t)sr, kq);
    return p;
}

// K order of a full tile.  A workgroup walks K upwards in its even-numbered
// tiles and downwards in its odd-numbered ones; the workgroups of one XCD
// run their n-th tiles together, so each round starts on the K stages the
// round before finished on, which are still in that XCD's L2.  Position i
// of the tile's K loop fetches stage base + i * step (in bytes of the
// stage's 128-byte tile); both are uniform scalars.
struct KOrder {
    int32_t base, step;
};
__host__ __device__ __forceinline__ KOrder k_order(int tile_index, int kt_count) {
    return (tile_index & 1) ? KOrder{(kt_count - 1) * 128, -128} : KOrder{0, 128};
}
__host__ __device__ __forceinline__ uint32_t stage_soff(const KOrder& o, int i) {
    return (uint32_t)(o.base + i * o.step);
}

// The quarter loop keeps kQDepth stages in flight and gives every stage the
// same body, so near the end of K (and in the prologue when K has fewer
// stages than that) it still issues loads for stages past the last one.
// Those loads fetch the last stage again instead (into a ring slot nobody
// reads any more): the stage a load at position s really fetches.
constexpr int kQDepth = 3;
__host__ __device__ __forceinline__ int qload_stage(int s, int kt_count) { return s < kt_count ? s : kt_count - 1; }

}  // namespace plan
}  // namespace fp4dit
