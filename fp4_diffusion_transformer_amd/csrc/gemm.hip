// Fused MXFP4 GEMM + epilogue for gfx950 (CDNA4).
//
// fal, epilogue-fusion section: the GEMM forms A . B tile by tile with the
// accumulators on chip, and the small ops that follow it (per-head RMSNorm
// on the attention path, gated SiLU in the FFN, the output cast) run on those
// accumulators before the single store, so the GEMM output never makes an
// extra HBM round trip.  KroQuant, "Deep analysis": both operands are MXFP4.
//
// Design (MI355X-first; the Blackwell tiling on the fal page is prior art):
// * Contraction on V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands (the
//   16x16x128 shape only reaches half the FP4 rate on this chip).  Its scale
//   operand carries one e8m0 byte per lane, exactly one MX block: lane l
//   holds row l%32 and the 32 K-elements of block l/32.
// * The GEMM is computed transposed, D = W . X^T: weight rows (output
//   channels) are the MFMA "A" operand, tokens the "B" operand, so a lane's
//   16 accumulators of a 32x32 block are 4 runs of 4 consecutive channels of
//   one token: a per-head sum needs one lane swap (l <-> l^32).
// * Workgroup tile 256 channels x 128 tokens, 4 waves of 128 x 64 (128 fp32
//   accumulators per lane).  With 76.5 KiB of LDS and <= 256 registers per
//   lane two workgroups share a CU, so one workgroup's epilogue overlaps the
//   other's main loop.
// * K is staged 128 at a time through a 3-deep LDS ring filled by the
//   direct-to-LDS global_load_lds_dwordx4 (no VGPR staging); stage kt+2 is in
//   flight while stage kt is multiplied.  One barrier per stage.  The three
//   ring slots are distinct __shared__ objects and the K loop is unrolled by
//   three, so every LDS access names its slot statically: the compiler can
//   then tell the fragment reads of stage kt+1 from the loads still landing
//   in stage kt+2 and does not drain all loads before each read.
// * LDS rows are 64 B (4 chunks of 16 B, one MX block each).  Chunk c of row
//   r is stored at c ^ ((r >> 2) & 3): each quarter-wave of a fragment read
//   (16 lanes = rows 0..15, 16 B each) then covers all 64 banks once.
// * K is permuted inside a stage: in K-step s lane group h takes MX block
//   2h + s, so a lane's two scale bytes of a stage are adjacent; one LDS
//   read fetches them and op_sel picks the byte.  Both operands use
//   the same permutation, so the sum over K is unchanged.
// * bf16 outputs go through LDS (after the main loop) so that every global
//   store writes whole row segments.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

constexpr int kBN = 256;               // channels per workgroup
constexpr int kBM = 128;               // tokens per workgroup
constexpr int kBK = 128;               // K elements per LDS stage
constexpr int kStages = 3;
constexpr int kRowBytes = kBK / 2;     // 64 bytes of codes per row per stage
constexpr int kScaleBytes = kBK / 32;  // 4 scale bytes per row per stage
constexpr int kWCodesOff = 0;
constexpr int kXCodesOff = kWCodesOff + kBN * kRowBytes;        // 16 KiB
constexpr int kWScalesOff = kXCodesOff + kBM * kRowBytes;       // +8 KiB
constexpr int kXScalesOff = kWScalesOff + kBN * kScaleBytes;    // +1 KiB
// Token scales: wave w loads rows 32w..32w+31 with all 64 lanes (lanes 32..63
// repeat them), so each wave owns a 256-byte slot whose first half is used.
constexpr int kStageBytes = kXScalesOff + 4 * 256;              // 26 KiB
constexpr int kLdsBytes = kStages * kStageBytes;                // 78 KiB
// Epilogue reuse of the ring: each wave stages 32 tokens x 256 B of bf16 at
// a time (8 KiB): waves 0..2 in stages 0..2, wave 3 in the second 8 KiB of
// stage 0; the per-token head sums (1 KiB) sit behind wave 1's region.
constexpr int kStageOutBytes = 8192;
constexpr int kRedOff = kStageOutBytes;
static_assert(2 * kStageOutBytes <= kStageBytes && kRedOff + 2 * kBM * 4 <= kStageBytes,
              "epilogue LDS does not fit");
constexpr int kDmaPerStage = 8;        // direct-to-LDS instructions per wave per stage

enum EpiKind { kEpiNone = 0, kEpiRmsNorm = 1, kEpiSwiglu = 2 };

struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    void* out;
    // rmsnorm
    int head_dim;
    int64_t n_norm;
    const float* norm_w;
    float eps;
    // swiglu requant
    uint8_t* out_codes;
    uint8_t* out_scales;
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding): vmcnt, expcnt, lgkmcnt.
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
    return (vm & 15) | ((exp & 7) << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

// Workgroup barrier of the K loop.  __syncthreads() would add a release
// fence, which drains every outstanding load -- including the direct-to-LDS
// loads of stage kt+2 that are meant to stay in flight.  Instead each wave
// waits explicitly (its stage-kt+1 loads landed: at most VM loads remain;
// its own LDS reads done) and then meets the others at s_barrier.  The empty
// asm statements keep the compiler from moving LDS accesses across it.
template <int VM>
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 7, 0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Per-lane byte offsets of the direct-to-LDS loads, fixed for the K loop (the
// stage advances the wave-uniform base pointers instead).
struct LoadPlan {
    uint32_t w_code[4], x_code[2];
    uint32_t w_scale, x_scale;
};

// Operands are MX_TILED: K stage kt of rows (2p, 2p+1) is one 128-byte code
// tile at ((p * K/128) + kt) * 128, and stage kt of 32 rows is one 128-byte
// scale tile, so every load fetches whole cache lines.
__device__ __forceinline__ uint32_t code_tile_off(uint32_t r, uint32_t kq) {
    return ((r >> 1) * kq) * 128 + (r & 1) * 64;
}
__device__ __forceinline__ uint32_t scale_tile_off(uint32_t r, uint32_t kq) {
    return ((r >> 5) * kq) * 128 + (r & 31) * 4;
}

__device__ __forceinline__ LoadPlan make_plan(const GemmArgs& g, int64_t n0, int64_t m0, int wave, int lane) {
    LoadPlan p;
    const uint32_t kq = (uint32_t)(g.K / 128);          // K stages (tiles per row pair / row block)
    const int rin = lane >> 2;                          // row within a 16-row group
    const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);  // chunk for physical slot lane & 3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (wave * 4 + j) * 16 + rin;
        p.w_code[j] = code_tile_off((uint32_t)(n0 + row), kq) + lchunk * 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = (wave * 2 + j) * 16 + rin;
        int64_t xr = m0 + row;
        xr = xr < g.M ? xr : g.M - 1;                   // ragged token tile: clamp, never stored
        p.x_code[j] = code_tile_off((uint32_t)xr, kq) + lchunk * 16;
    }
    p.w_scale = scale_tile_off((uint32_t)(n0 + wave * 64 + lane), kq);
    int64_t xr = m0 + wave * 32 + (lane & 31);          // lanes 32..63 repeat lanes 0..31
    xr = xr < g.M ? xr : g.M - 1;
    p.x_scale = scale_tile_off((uint32_t)xr, kq);
    return p;
}

// Enqueue the 8 direct-to-LDS loads of K stage kt into `stage` (this wave's share).
__device__ __forceinline__ void issue_stage(uint8_t* stage, const GemmArgs& g, const LoadPlan& p, int kt,
                                            int wave, int lane) {
    const uint8_t* wc = g.b_codes + (int64_t)kt * 128;
    const uint8_t* xc = g.a_codes + (int64_t)kt * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_global_load_lds(wc + p.w_code[j], (lds_void*)(stage + kWCodesOff + (wave * 4 + j) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds(xc + p.x_code[j], (lds_void*)(stage + kXCodesOff + (wave * 2 + j) * 1024),
                                         16, 0, 0);
    __builtin_amdgcn_global_load_lds(g.b_scales + (int64_t)kt * 128 + p.w_scale,
                                     (lds_void*)(stage + kWScalesOff + wave * 256), 4, 0, 0);
    // 128 token rows of scales: 32 per wave, into the wave's 256-byte slot
    __builtin_amdgcn_global_load_lds(g.a_scales + (int64_t)kt * 128 + p.x_scale,
                                     (lds_void*)(stage + kXScalesOff + wave * 256), 4, 0, 0);
}

struct Frags {
    v4i w[4], x[2];
};

// Fragment reads of K-step s: lane group h takes MX block 2h + s of the stage.
__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* stage, int wn, int wm, int r32, int h,
                                           int s) {
    const int chunk = ((2 * h + s) ^ ((r32 >> 2) & 3)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.w[i] = *reinterpret_cast<const v4i*>(stage + kWCodesOff + (wn * 128 + i * 32 + r32) * kRowBytes + chunk);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        f.x[i] = *reinterpret_cast<const v4i*>(stage + kXCodesOff + (wm * 64 + i * 32 + r32) * kRowBytes + chunk);
}

// Scale bytes 2h, 2h+1 of every fragment row (byte s serves K-step s),
// read as the row's whole dword: a 16-bit LDS read here makes the compiler
// wait for every load still in flight (it cannot tell it apart from the
// loads landing in the other ring slots), a 32-bit one does not.
__device__ __forceinline__ void read_scales(uint32_t* wsc, uint32_t* xsc, const uint8_t* stage, int wn, int wm,
                                            int r32, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        wsc[i] = *reinterpret_cast<const uint32_t*>(stage + kWScalesOff + (wn * 128 + i * 32 + r32) * kScaleBytes) >> (16 * h);
#pragma unroll
    for (int i = 0; i < 2; ++i)   // token row wm*64 + i*32 + r32 sits in slot (2wm + i) at r32*4
        xsc[i] = *reinterpret_cast<const uint32_t*>(stage + kXScalesOff + (wm * 2 + i) * 256 + r32 * kScaleBytes) >> (16 * h);
}

template <int S>
__device__ __forceinline__ void mfma_step(v16f (&acc)[4][2], const Frags& f, const uint32_t* wsc,
                                          const uint32_t* xsc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v8i a = {f.w[i][0], f.w[i][1], f.w[i][2], f.w[i][3], 0, 0, 0, 0};
            const v8i b = {f.x[j][0], f.x[j][1], f.x[j][2], f.x[j][3], 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, S, (int)wsc[i],
                                                                        S, (int)xsc[j]);
        }
}

// Scheduling of one K-step: its 8 MFMAs interleaved with the 6 fragment
// reads of the next K-step and, in the first K-step of a stage, with the 8
// direct-to-LDS loads of stage kt+2 (masks: 0x008 MFMA, 0x020 VMEM read,
// 0x100 DS read).
__device__ __forceinline__ void sched_step0() {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void sched_step1() {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Map the linear workgroup id to a (token tile, channel tile).  Workgroups
// are dispatched round-robin over the 8 XCDs; consecutive remapped ids land
// on one XCD and walk a band of 8 token tiles across the channel tiles, so
// the workgroups an XCD runs together share operand rows in its L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t nwg, int64_t tiles_n, int64_t tiles_m,
                                        int64_t& tm, int64_t& tn) {
    int64_t b = bid;
    if ((nwg & 7) == 0) b = (bid & 7) * (nwg >> 3) + (bid >> 3);
    constexpr int64_t kGroupM = 8;
    const int64_t per_group = kGroupM * tiles_n;
    const int64_t group = b / per_group;
    const int64_t first = group * kGroupM;
    const int64_t gm = (tiles_m - first) < kGroupM ? (tiles_m - first) : kGroupM;
    const int64_t in = b - group * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

// Store 32 tokens x 8Q bf16 columns of this wave through its LDS region so
// that every global store writes whole row segments.  vals(q, v) gives the
// lane's 4 fp32 values of 8-column chunk q (half h) for token tok0 + r32.
// In LDS, chunk q of token row t sits at q ^ (t % Q) and its two halves are
// swapped on every other group of Q rows, so both the 8-byte writes and the
// 16-byte row reads spread over all banks.  Called by all 4 waves together.
template <int Q, typename F>
__device__ __forceinline__ void store_bf16_half(uint8_t* region, F vals, uint16_t* out, int64_t ld,
                                                int64_t tok0, int64_t col0, int64_t M, int r32, int h, int lane) {
    constexpr int kRow = Q * 16;                       // bytes per token row
    const int t = r32;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        float v[4];
        vals(q, v);
        v2u o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        const int off = t * kRow + ((q ^ (t % Q)) * 16) + ((h ^ ((t / Q) & 1)) * 8);
        *reinterpret_cast<v2u*>(region + off) = o;
    }
    __syncthreads();
    constexpr int kRowsPerInst = 64 / Q;               // Q lanes x 16 B per token row
#pragma unroll
    for (int it = 0; it < 32 / kRowsPerInst; ++it) {
        const int tr = it * kRowsPerInst + lane / Q;
        const int q = lane % Q;
        v4u v = *reinterpret_cast<const v4u*>(region + tr * kRow + ((q ^ (tr % Q)) * 16));
        if ((tr / Q) & 1) v = (v4u){v[2], v[3], v[0], v[1]};
        const int64_t tok = tok0 + tr;
        if (tok < M) *reinterpret_cast<v4u*>(out + tok * ld + col0 + q * 8) = v;
    }
    __syncthreads();
}

// One K stage of the main loop on ring slot `cur` (static).  ISSUE: also
// enqueue the loads of stage kt+2 into slot `fill`; NEXT: prefetch the scales
// and first fragments of stage kt+1 from slot `nxt` after the barrier.
template <bool ISSUE, bool NEXT>
__device__ __forceinline__ void k_stage(v16f (&acc)[4][2], Frags& f0, Frags& f1, uint32_t* wsc, uint32_t* xsc,
                                        uint8_t* cur, uint8_t* nxt, uint8_t* fill, const GemmArgs& g,
                                        const LoadPlan& plan, int kt, int wave, int lane, int wn, int wm, int r32,
                                        int h) {
    uint32_t wsn[4], xsn[2];
    if (ISSUE) issue_stage(fill, g, plan, kt + 2, wave, lane);
    read_frags(f1, cur, wn, wm, r32, h, 1);
    mfma_step<0>(acc, f0, wsc, xsc);
    if (ISSUE) sched_step0(); else sched_step1();
    if (NEXT) {
        // Stage kt+1 landed (only stage kt+2's loads may remain) and this
        // stage's fragments are in registers: after the barrier stage kt+1
        // may be read and stage kt overwritten.
        ring_barrier<ISSUE ? kDmaPerStage : 0>();
        read_scales(wsn, xsn, nxt, wn, wm, r32, h);
        read_frags(f0, nxt, wn, wm, r32, h, 0);
    }
    mfma_step<1>(acc, f1, wsc, xsc);
    if (NEXT) {
        sched_step1();
#pragma unroll
        for (int i = 0; i < 4; ++i) wsc[i] = wsn[i];
#pragma unroll
        for (int i = 0; i < 2; ++i) xsc[i] = xsn[i];
    }
}

template <int EPI, bool OUT_BF16, int REM>
__global__ __launch_bounds__(256, 2) void gemm_fp4_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t ring2[kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;              // channel half of the workgroup tile (128 channels)
    const int wm = wave >> 1;             // token half (64 tokens)
    const int64_t tiles_n = g.N / kBN;
    const int64_t tiles_m = (g.M + kBM - 1) / kBM;
    int64_t tm, tn;
    tile_of(blockIdx.x, (int64_t)gridDim.x, tiles_n, tiles_m, tm, tn);
    const int64_t n0 = tn * kBN;
    const int64_t m0 = tm * kBM;
    const int kt_count = (int)(g.K / kBK);   // even and >= 2 (K % 256 == 0)

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

    const int r32 = lane & 31;
    const int h = lane >> 5;

    // Ring slot of stage j is (j + OFF) % 3 with OFF chosen so that the
    // REM = (kt_count - 2) % 3 stages before the unrolled loop absorb the
    // remainder: the loop then always starts on slot 0 and the last two
    // stages always sit in slots 0 and 1, all known at compile time.
    constexpr int OFF = (3 - REM) % 3;
    uint8_t* const slots[3] = {ring0, ring1, ring2};
    const LoadPlan plan = make_plan(g, n0, m0, wave, lane);
    issue_stage(slots[OFF % 3], g, plan, 0, wave, lane);
    issue_stage(slots[(OFF + 1) % 3], g, plan, 1, wave, lane);
    ring_barrier<kDmaPerStage>();                    // stage 0 landed

    Frags f0, f1;
    uint32_t wsc[4], xsc[2];
    read_scales(wsc, xsc, slots[OFF % 3], wn, wm, r32, h);
    read_frags(f0, slots[OFF % 3], wn, wm, r32, h, 0);

#define FP4DIT_STAGE(ISSUE, NEXT, CUR, NXT, FILL, KT) \
    k_stage<ISSUE, NEXT>(acc, f0, f1, wsc, xsc, slots[CUR], slots[NXT], slots[FILL], g, plan, KT, wave, lane, \
                         wn, wm, r32, h)
    // stages 0 .. REM-1 (each issues the loads of stage j + 2)
    if (REM >= 1) FP4DIT_STAGE(true, true, (OFF + 0) % 3, (OFF + 1) % 3, (OFF + 2) % 3, 0);
    if (REM >= 2) FP4DIT_STAGE(true, true, (OFF + 1) % 3, (OFF + 2) % 3, (OFF + 0) % 3, 1);
    // stages REM .. kt_count - 3, three at a time, on slots 0, 1, 2
    for (int kt = REM; kt < kt_count - 2; kt += 3) {
        FP4DIT_STAGE(true, true, 0, 1, 2, kt);
        FP4DIT_STAGE(true, true, 1, 2, 0, kt + 1);
        FP4DIT_STAGE(true, true, 2, 0, 1, kt + 2);
    }
    // the last two stages: no more loads
    FP4DIT_STAGE(false, true, 0, 1, 2, kt_count - 2);
    FP4DIT_STAGE(false, false, 1, 2, 0, kt_count - 1);
#undef FP4DIT_STAGE
    __syncthreads();                      // the epilogue reuses the LDS ring

    // ------------------------------------------------------------ epilogue --
    // acc[nb][mb][i]: channel n0 + wn*128 + nb*32 + 8*(i/4) + 4h + i%4,
    //                 token   m0 + wm*64 + mb*32 + r32.
    const int64_t cbase = n0 + wn * 128;
    const int64_t tok0 = m0 + wm * 64;
    uint8_t* region = wave == 0 ? ring0 : wave == 1 ? ring1 : wave == 2 ? ring2 : ring0 + kStageOutBytes;
    if (EPI == kEpiNone || EPI == kEpiRmsNorm) {
        float rstd[2] = {1.f, 1.f};
        bool norm = false;
        if (EPI == kEpiRmsNorm) {
            float* red = reinterpret_cast<float*>(ring1 + kRedOff);  // [2 wn][128 tokens]
            float ss[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                float s = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s += acc[nb][mb][i] * acc[nb][mb][i];
                ss[mb] = sum_xor32(s);
            }
            if (g.head_dim == 256) {                      // head = both channel halves
                if (h == 0) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) red[wn * kBM + wm * 64 + mb * 32 + r32] = ss[mb];
                }
                __syncthreads();
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) ss[mb] += red[(1 - wn) * kBM + wm * 64 + mb * 32 + r32];
            }
            const int64_t head0 = g.head_dim == 256 ? n0 : cbase;
            norm = head0 < g.n_norm;
            const float inv_d = 1.0f / (float)g.head_dim;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) rstd[mb] = rsqrtf(ss[mb] * inv_d + g.eps);
        }
        v4f wv[4][4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                wv[nb][a] = (v4f){1.f, 1.f, 1.f, 1.f};
                if (EPI == kEpiRmsNorm && norm)
                    wv[nb][a] = *reinterpret_cast<const v4f*>(g.norm_w + cbase + nb * 32 + 8 * a + 4 * h);
            }
        auto vals = [&](int q, int mb, float* v) {
            const int nb = q >> 2, a = q & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = (EPI == kEpiRmsNorm && norm) ? acc[nb][mb][4 * a + r] * rstd[mb] * wv[nb][a][r]
                                                    : acc[nb][mb][4 * a + r];
        };
        if (OUT_BF16) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                store_bf16_half<16>(region, [&](int q, float* v) { vals(q, mb, v); }, static_cast<uint16_t*>(g.out),
                                    g.N, tok0 + mb * 32, cbase, g.M, r32, h, lane);
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int64_t tok = tok0 + mb * 32 + r32;
                if (tok >= g.M) continue;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    float v[4];
                    vals(q, mb, v);
                    *reinterpret_cast<v4f*>(static_cast<float*>(g.out) + tok * g.N + cbase + (q >> 2) * 32 +
                                            8 * (q & 3) + 4 * h) = (v4f){v[0], v[1], v[2], v[3]};
                }
            }
        }
    }

    if (EPI == kEpiSwiglu) {
        // Channel blocks alternate gate / up (interleave group 32): block 2p
        // of the wave holds gate outputs and block 2p+1 the matching up
        // outputs cbase/2 + 32p + 8a + 4h + r.
        const int64_t nh = g.N / 2;
        const int64_t ob0 = cbase / 2;
        float hv[2][2][16];                   // [p][mb][4a + r]
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[p][mb][i] = silu_f(acc[2 * p][mb][i]) * acc[2 * p + 1][mb][i];
        if (g.out != nullptr) {
            if (OUT_BF16) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    store_bf16_half<8>(region, [&](int q, float* v) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) v[r] = hv[q >> 2][mb][4 * (q & 3) + r];
                    }, static_cast<uint16_t*>(g.out), nh, tok0 + mb * 32, ob0, g.M, r32, h, lane);
            } else {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int64_t tok = tok0 + mb * 32 + r32;
                    if (tok >= g.M) continue;
#pragma unroll
                    for (int p = 0; p < 2; ++p)
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            *reinterpret_cast<v4f*>(static_cast<float*>(g.out) + tok * nh + ob0 + 32 * p + 8 * a +
                                                    4 * h) =
                                (v4f){hv[p][mb][4 * a], hv[p][mb][4 * a + 1], hv[p][mb][4 * a + 2], hv[p][mb][4 * a + 3]};
                }
            }
        }
        if (g.out_codes != nullptr) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int64_t tok = tok0 + mb * 32 + r32;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    uint32_t amax = 0u;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const uint32_t a = __float_as_uint(hv[p][mb][i]) & 0x7FFFFFFFu;
                        amax = a > amax ? a : amax;
                    }
                    amax = max_xor32_u(amax);
                    const uint32_t sc = e8m0_from_amax_bits(amax);
                    uint32_t c16[4];                  // codes of outputs 8a+4h .. +3
#pragma unroll
                    for (int a = 0; a < 4; ++a) c16[a] = sc == 0xFFu ? 0u : e2m1_pack4(&hv[p][mb][4 * a], sc);
                    // lane h=0 stores bytes 0..7 of the block (outputs 0..15),
                    // lane h=1 bytes 8..15; each needs two halves from its partner.
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
                    if (tok < g.M) {                  // MX_TILED output, ready for the next GEMM
                        const int64_t blk = ob0 / 32 + p;
                        *reinterpret_cast<v2u*>(g.out_codes + tiled_code_off(tok, blk * 32, nh) + h * 8) = st;
                        if (h == 0) g.out_scales[tiled_scale_off(tok, blk, nh)] = (uint8_t)sc;
                    }
                }
            }
        }
    }
}

template <int EPI, bool OUT_BF16>
void launch_rem(const GemmArgs& g, dim3 grid, hipStream_t stream) {
    switch ((g.K / kBK - 2) % 3) {
        case 0: hipLaunchKernelGGL((gemm_fp4_kernel<EPI, OUT_BF16, 0>), grid, dim3(256), 0, stream, g); break;
        case 1: hipLaunchKernelGGL((gemm_fp4_kernel<EPI, OUT_BF16, 1>), grid, dim3(256), 0, stream, g); break;
        default: hipLaunchKernelGGL((gemm_fp4_kernel<EPI, OUT_BF16, 2>), grid, dim3(256), 0, stream, g); break;
    }
}

template <int EPI>
void launch_epi(const GemmArgs& g, bool out_bf16, dim3 grid, hipStream_t stream) {
    if (out_bf16) {
        launch_rem<EPI, true>(g, grid, stream);
    } else {
        launch_rem<EPI, false>(g, grid, stream);
    }
}

hipError_t launch_gemm(const GemmArgs& g, int epi, bool out_bf16, hipStream_t stream) {
    const int64_t tiles = (g.N / kBN) * ((g.M + kBM - 1) / kBM);
    const dim3 grid((unsigned)tiles);
    switch (epi) {
        case kEpiNone: launch_epi<kEpiNone>(g, out_bf16, grid, stream); break;
        case kEpiRmsNorm: launch_epi<kEpiRmsNorm>(g, out_bf16, grid, stream); break;
        default: launch_epi<kEpiSwiglu>(g, out_bf16, grid, stream); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_none(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                            const uint8_t* bc, const uint8_t* bs, void* out, bool out_bf16,
                            hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out;
    return launch_gemm(g, kEpiNone, out_bf16, stream);
}

hipError_t launch_gemm_rmsnorm(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                               const uint8_t* bc, const uint8_t* bs, int head_dim, int64_t n_norm,
                               const float* norm_w, float eps, void* out, bool out_bf16,
                               hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out;
    g.head_dim = head_dim; g.n_norm = n_norm; g.norm_w = norm_w; g.eps = eps;
    return launch_gemm(g, kEpiRmsNorm, out_bf16, stream);
}

hipError_t launch_gemm_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                              const uint8_t* bc, const uint8_t* bs, void* out, bool out_bf16,
                              uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out;
    g.out_codes = out_codes; g.out_scales = out_scales;
    return launch_gemm(g, kEpiSwiglu, out_bf16, stream);
}

}  // namespace fp4dit
