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
// * Workgroup tile 256 channels x 256 tokens, 4 waves of 128 x 128: 256 fp32
//   accumulators per lane, held in the accumulation registers, so one wave
//   fills a SIMD's register file and a CU runs one workgroup.  The large wave
//   tile is what bounds the LDS traffic: per K-step a wave reads 8 KiB of
//   fragments for 16 MFMAs, and the operands enter LDS once per 256 x 256
//   tile.  With 64 B of codes per row per 128-K stage, LDS (not HBM, not L2
//   latency) is the shared resource the main loop has to spare.
// * K is staged 128 at a time through a kRing-deep LDS ring filled by the
//   direct-to-LDS global_load_lds_dwordx4 (no VGPR staging); stage
//   kt + kRing - 1 is in flight while stage kt is multiplied.  One barrier
//   per stage.  The ring slots are distinct __shared__ objects and the K
//   loop is unrolled by kRing, so every LDS access names its slot
//   statically: the compiler then tells the fragment reads of stage kt+1
//   from the loads still landing in later slots and does not drain all
//   loads before each read.
// * LDS rows are 64 B (4 chunks of 16 B, one MX block each).  Chunk c of row
//   r is stored at c ^ ((r >> 2) & 3): each quarter-wave of a fragment read
//   (16 lanes = rows 0..15, 16 B each) then covers all 64 banks once.
// * K is permuted inside a stage: in K-step s lane group h takes MX block
//   2h + s, so a lane's two scale bytes of a stage are adjacent; one LDS
//   read fetches them and op_sel picks the byte.  Both operands use
//   the same permutation, so the sum over K is unchanged.
// * Persistent grid, one workgroup per CU, tiles in an XCD-aware order; a
//   workgroup's K loop alternates direction from tile to tile (up, down,
//   ...), so each round of tiles starts on the K stages the previous round
//   left in the XCD's L2.  Below, "stage kt" is position kt of the tile's
//   K order; plan::stage_soff gives the stage it fetches.
// * bf16 outputs go through LDS (after the main loop) so that every global
//   store writes whole row segments.
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "gemm_plan.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

constexpr int kBN = 256;               // channels per workgroup
constexpr int kBM = 256;               // tokens per workgroup
constexpr int kBK = 128;               // K elements per LDS stage
constexpr int kRing = 3;               // LDS ring depth (stages)
constexpr int kRowBytes = kBK / 2;     // 64 bytes of codes per row per stage
constexpr int kScaleBytes = kBK / 32;  // 4 scale bytes per row per stage
constexpr int kWCodesOff = 0;
constexpr int kXCodesOff = kWCodesOff + kBN * kRowBytes;        // 16 KiB
constexpr int kWScalesOff = kXCodesOff + kBM * kRowBytes;       // +16 KiB
constexpr int kXScalesOff = kWScalesOff + kBN * kScaleBytes;    // +1 KiB
constexpr int kStageBytes = kXScalesOff + kBM * kScaleBytes;    // 34 KiB
// Epilogue use of the one ring slot the next tile's prefetch leaves free:
// each wave stages 32 tokens x 256 B of bf16 at a time in its own region of
// 32 padded rows (8.5 KiB); the per-token head sums of a 256-wide head (2 KiB)
// are exchanged at the start of the slot before any wave stages its rows.
constexpr int kStageOutBytes = 32 * (16 * 16 + 16);
constexpr int kRedOff = 0;
static_assert(4 * kStageOutBytes <= kStageBytes && kRedOff + 2 * kBM * 4 <= kStageBytes,
              "epilogue LDS does not fit");
constexpr int kDmaPerStage = 10;       // direct-to-LDS instructions per wave per stage
constexpr int kDmaEarly = 8;           // of them issued before the stage's barrier

enum EpiKind { kEpiNone = 0, kEpiRmsNorm = 1, kEpiSwiglu = 2, kEpiSwigluTransform = 3 };
// What the `out` array receives (a compile-time choice, so a kernel holds
// only the store code it runs): nothing (SwiGLU requant only), bf16, fp32.
enum OutKind { kOutNone = 0, kOutBf16 = 1, kOutF32 = 2 };

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
    // block transform of the SwiGLU output before the requant: T [n_t][32][32]
    const uint16_t* t;
    int64_t n_t;
};

typedef short v8s __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void;

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1 (device
// code; static_for_host for the launchers).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}
template <int B, int E, typename F>
void static_for_host(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for_host<B + 1, E>(f);
    }
}

// s_waitcnt immediate (gfx9 encoding): vmcnt, expcnt, lgkmcnt.
constexpr int waitcnt_imm(int vm, int exp, int lgkm) {
    return (vm & 15) | ((exp & 7) << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

// Workgroup barrier of the K loop.  __syncthreads() would add a release
// fence, which drains every outstanding load -- including the direct-to-LDS
// loads of later stages that are meant to stay in flight.  Instead each wave
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

// Orders the LDS writes and reads of one wave's lanes (a wave's LDS
// operations execute in order; this only stops the compiler from moving
// them).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// A wave-uniform 32-bit value the compiler may not hoist or fold: LDS
// destinations derived from it cost one scalar add per load instead of one
// live scalar register per (ring slot, load).
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t x) {
    asm volatile("" : "+s"(x));
    return x;
}

// This lane's index in the wave (v_mbcnt over the full mask), recomputed at
// every call: per-lane values derived from it are formed where they are used
// instead of being kept live (and spilled) across the whole tile loop.
__device__ __forceinline__ int fresh_lane_id() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return (int)l;
}

using plan::LoadPlan;
using plan::QPlan;
using plan::make_plan;
using plan::make_qplan;

// Buffer descriptors of the four operand arrays (scalar registers, set up
// once): every load of a stage then adds the stage's scalar offset
// (stage * 128) to its fixed per-lane offset.  The record counts are the
// arrays' sizes.
struct Operands {
    __amdgpu_buffer_rsrc_t wc, xc, ws, xs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t* p, int64_t bytes) {
    constexpr int kRawDword = 0x00020000;               // untyped 32-bit data format, no swizzle
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)bytes, kRawDword);
}

__device__ __forceinline__ Operands make_operands(const GemmArgs& g) {
    Operands o;
    o.wc = buffer_rsrc(g.b_codes, plan::code_bytes(g.N, g.K));
    o.xc = buffer_rsrc(g.a_codes, plan::code_bytes(g.M, g.K));
    o.ws = buffer_rsrc(g.b_scales, plan::scale_bytes(g.N, g.K));
    o.xs = buffer_rsrc(g.a_scales, plan::scale_bytes(g.M, g.K));
    return o;
}

// Enqueue the 10 direct-to-LDS loads of the K stage at scalar offset soff
// (stage * 128; this wave's share).  codes / scales: LDS byte addresses of
// this wave's part of the stage's code and scale areas (stage + wave * 4096,
// stage + wave * 256).
__device__ __forceinline__ void issue_stage(uint32_t codes, uint32_t scales, const Operands& o, const LoadPlan& p,
                                            uint32_t soff) {
    auto lds = [](uint32_t a) { return (lds_void*)(uintptr_t)a; };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.wc, lds(codes + kWCodesOff + j * 1024), 16, p.w_code[j], soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xc, lds(codes + kXCodesOff + j * 1024), 16, p.x_code[j], soff, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.ws, lds(scales + kWScalesOff), 4, p.w_scale, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xs, lds(scales + kXScalesOff), 4, p.x_scale, soff, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// Load l (0..9) of a stage: 0..3 weight codes, 4..7 token codes, 8 weight
// scales, 9 token scales (the same loads as issue_stage, one at a time; l is
// a compile-time constant at every call, so the switch folds away).
__device__ __forceinline__ void issue_load(int l, uint32_t codes, uint32_t scales, const Operands& o,
                                           const LoadPlan& p, uint32_t soff) {
    auto lds = [](uint32_t a) { return (lds_void*)(uintptr_t)a; };
    switch (l) {
        case 0: case 1: case 2: case 3:
            __builtin_amdgcn_raw_ptr_buffer_load_lds(o.wc, lds(codes + kWCodesOff + l * 1024), 16, p.w_code[l], soff, 0,
                                                     0);
            break;
        case 4: case 5: case 6: case 7:
            __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xc, lds(codes + kXCodesOff + (l - 4) * 1024), 16, p.x_code[l - 4],
                                                     soff, 0, 0);
            break;
        case 8:
            __builtin_amdgcn_raw_ptr_buffer_load_lds(o.ws, lds(scales + kWScalesOff), 4, p.w_scale, soff, 0, 0);
            break;
        default:
            __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xs, lds(scales + kXScalesOff), 4, p.x_scale, soff, 0, 0);
            break;
    }
}

// Whole-stage prefetch outside the K loop (prologue of a tile).
__device__ __forceinline__ void issue_stage_at(uint8_t* stage, const Operands& o, const LoadPlan& p, uint32_t soff,
                                               int wave) {
    const uint32_t codes = opaque_sgpr(lds_addr(stage) + wave * 4096);
    const uint32_t scales = opaque_sgpr(lds_addr(stage) + wave * 256);
    issue_stage(codes, scales, o, p, soff);
}

struct Frags {
    v4i w[4], x[4];
};

// Fragment reads of K-step s: lane group h takes MX block 2h + s of the stage.
__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* stage, int wn, int wm, int r32, int h,
                                           int s) {
    const int chunk = ((2 * h + s) ^ ((r32 >> 2) & 3)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.w[i] = *reinterpret_cast<const v4i*>(stage + kWCodesOff + (wn * 128 + i * 32 + r32) * kRowBytes + chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.x[i] = *reinterpret_cast<const v4i*>(stage + kXCodesOff + (wm * 128 + i * 32 + r32) * kRowBytes + chunk);
}

// Scale bytes 2h, 2h+1 of every fragment row (byte s serves K-step s, picked
// by op_sel), read as one 16-bit value so that no per-lane shift is needed.
__device__ __forceinline__ void read_scales(uint32_t* wsc, uint32_t* xsc, const uint8_t* stage, int wn, int wm,
                                            int r32, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        wsc[i] = *reinterpret_cast<const uint16_t*>(stage + kWScalesOff + (wn * 128 + i * 32 + r32) * kScaleBytes + 2 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xsc[i] = *reinterpret_cast<const uint16_t*>(stage + kXScalesOff + (wm * 128 + i * 32 + r32) * kScaleBytes + 2 * h);
}

__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Map the linear workgroup id to a (token tile, channel tile).  Workgroups
// are dispatched round-robin over the 8 XCDs; consecutive remapped ids land
// on one XCD and walk a band of 8 token tiles across the channel tiles, so
// the workgroups an XCD runs together share operand rows in its L2.
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_n, int tiles_m, int& tm, int& tn) {
    int b = bid;
    if ((nwg & 7) == 0) b = (bid & 7) * (nwg >> 3) + (bid >> 3);
    constexpr int kGroupM = 8;
    const int per_group = kGroupM * tiles_n;
    const int group = b / per_group;
    const int first = group * kGroupM;
    const int gm = (tiles_m - first) < kGroupM ? (tiles_m - first) : kGroupM;
    const int in = b - group * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

// Store 32 tokens x 8Q bf16 columns of this wave through its LDS region so
// that every global store writes whole row segments.  vals(q, v) gives the
// lane's 4 fp32 values of 8-column chunk q (half h) for token tok0 + r32.
// Token rows sit kRowPad = 16Q + 16 bytes apart: the 16-byte pad rotates
// consecutive rows by four banks.  A lane holds half of each 16-byte chunk
// (4 of its 8 columns; its partner lane l ^ 32 the other half), and the 16
// lanes of a quarter-wave hold 16 different rows of one half, so 8-byte
// writes of the halves put rows r and r + 8 on the same banks
// (SQ_LDS_BANK_CONFLICT: about 12% of the RMSNorm GEMMs' LDS-active cycles).
// Instead, for each pair of chunks (2p, 2p + 1) one v_permlane32_swap per
// dword hands lane h = 0 the whole chunk 2p and lane h = 1 the whole chunk
// 2p + 1: one 16-byte write per lane and pair, every group of 8 lanes on
// distinct banks, and half as many LDS writes.  The row reads are 16 bytes
// per lane, conflict-free with the same pad.  All accesses of a lane share
// one base address (immediate offsets).  Only this wave touches `region`
// (32 * kRowPad bytes).
template <int Q>
constexpr int row_pad_bytes() { return Q * 16 + 16; }

template <int Q, typename F>
__device__ __forceinline__ void store_bf16_half(uint8_t* region, F vals, uint16_t* out, int64_t ld,
                                                int64_t tok0, int64_t col0, int64_t M, int r32, int h, int lane) {
    static_assert(Q % 2 == 0, "chunks go in pairs");
    constexpr int kRowPad = row_pad_bytes<Q>();
    uint8_t* wbase = region + r32 * kRowPad + h * 16;
#pragma unroll
    for (int p = 0; p < Q / 2; ++p) {
        float va[4], vb[4];
        vals(2 * p, va);
        vals(2 * p + 1, vb);
        // this lane's 4 columns (half h) of chunks 2p (a) and 2p + 1 (b)
        const uint32_t a0 = pack_bf16x2(va[0], va[1]), a1 = pack_bf16x2(va[2], va[3]);
        const uint32_t b0 = pack_bf16x2(vb[0], vb[1]), b1 = pack_bf16x2(vb[2], vb[3]);
        // swap(a, b): lanes 0..31 keep a and receive the partner's a, lanes
        // 32..63 receive the partner's b and keep b -- i.e. {x[0], y[0]} is
        // the whole chunk 2p + h as (low 4 columns, high 4 columns)
        const auto x = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const v4u o = {x[0], y[0], x[1], y[1]};
        *reinterpret_cast<v4u*>(wbase + p * 32) = o;
    }
    wave_lds_fence();
    // Read back all of the wave's rows before the first store: one wait for
    // the LDS instead of one per row.  The stores go through a descriptor
    // whose record count ends at token row M, so the hardware drops rows past
    // it without a branch per row; 32 rows x ld bf16 is far below 2^31 bytes
    // (ld * K/2 < 2^31 with K >= 256).
    constexpr int kRowsPerInst = 64 / Q;               // Q lanes x 16 B per token row
    constexpr int kIts = 32 / kRowsPerInst;
    const int q = lane % Q;
    const uint8_t* rbase = region + (lane / Q) * kRowPad + q * 16;
    v4u rows[kIts];
#pragma unroll
    for (int it = 0; it < kIts; ++it) rows[it] = *reinterpret_cast<const v4u*>(rbase + it * kRowsPerInst * kRowPad);
    // all rows held at once: without this the register allocator (the file
    // is nearly full here) reuses one row's registers for the next, which
    // puts a full LDS round trip before every store
#pragma unroll
    for (int it = 0; it < kIts; ++it) asm volatile("" : "+v"(rows[it]));
    const int64_t valid = M - tok0 < 0 ? 0 : (M - tok0 < 32 ? M - tok0 : 32);
    const __amdgpu_buffer_rsrc_t o =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(out + tok0 * ld + col0), valid * ld * 2);
    const int row_bytes = (int)ld * 2;
    const int off = (lane / Q) * row_bytes + q * 16;
    // Non-temporal (cache policy nt): the output is written once and not read
    // back by this kernel.  Measured with four output buffers in rotation
    // (more than the last-level cache holds): 4096x9216x3072 RMSNorm GEMM
    // 70.6 -> 67.3 us, 4096x12288x4096 within 1%; with one output buffer,
    // which stays cache-resident, within 1% for both.  The SwiGLU requant
    // stores timed the same either way and keep the default policy.
    constexpr int kStoreNt = 2;
#pragma unroll
    for (int it = 0; it < kIts; ++it)
        __builtin_amdgcn_raw_buffer_store_b128(rows[it], o, off + it * kRowsPerInst * row_bytes, 0, kStoreNt);
    wave_lds_fence();
}

// One MFMA of K-step S: accumulator block (i, j) = weight fragment i x token
// fragment j.
template <int S>
__device__ __forceinline__ void mfma_one(v16f& acc, const v4i& w, const v4i& x, uint32_t ws, uint32_t xs) {
    const v8i a = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
    const v8i b = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, S, (int)ws, S, (int)xs);
}

// Fragment r (0..3 weight rows i = r, 4..7 token rows j = r - 4) of K-step s.
template <int R>
__device__ __forceinline__ void read_frag(Frags& f, const uint8_t* stage, int wn, int wm, int r32, int h, int s) {
    const int chunk = ((2 * h + s) ^ ((r32 >> 2) & 3)) * 16;
    if constexpr (R < 4)
        f.w[R] = *reinterpret_cast<const v4i*>(stage + kWCodesOff + (wn * 128 + R * 32 + r32) * kRowBytes + chunk);
    else
        f.x[R - 4] = *reinterpret_cast<const v4i*>(stage + kXCodesOff + (wm * 128 + (R - 4) * 32 + r32) * kRowBytes +
                                                   chunk);
}

// Scale pair r (0..3 weight rows, 4..7 token rows) of a stage: bytes 2h, 2h+1
// of the row (byte s serves K-step s, picked by op_sel), one 16-bit read.
template <int R>
__device__ __forceinline__ void read_scale(uint32_t* wsc, uint32_t* xsc, const uint8_t* stage, int wn, int wm, int r32,
                                           int h) {
    if constexpr (R < 4)
        wsc[R] = *reinterpret_cast<const uint16_t*>(stage + kWScalesOff + (wn * 128 + R * 32 + r32) * kScaleBytes + 2 * h);
    else
        xsc[R - 4] = *reinterpret_cast<const uint16_t*>(stage + kXScalesOff + (wm * 128 + (R - 4) * 32 + r32) * kScaleBytes +
                                                        2 * h);
}

// One K stage of the main loop on ring slot `cur`, scheduled by hand (each
// sched_barrier pins the instructions issued since the previous one):
// * K-step 0: MFMA n on the fragments read one step earlier, with (ISSUE)
//   load n/2 of stage kt + kRing - 1 on every even n -- kDmaEarly loads --
//   and the read of second-step fragment n (n < 8);
// * barrier (NEXT): this wave's stage-kt+1 loads landed (at most VM loads
//   remain in flight) and every wave is done with stage kt;
// * K-step 1: the last kDmaPerStage - kDmaEarly loads go out with MFMAs 6..,
//   and the 8 scale then 8 fragment reads of stage kt+1 one per MFMA.
// Measured against packing the loads into the first 10 slots, reads into the
// first 8 of K-step 1, or loading after the barrier: about 2% faster.
template <bool ISSUE, bool NEXT, int VM, bool MB_MAJOR = false>
__device__ __forceinline__ void k_stage(v16f (&acc)[4][4], Frags& f0, Frags& f1, uint32_t* wsc, uint32_t* xsc,
                                        uint8_t* cur_, uint8_t* nxt_, uint8_t* fill, const Operands& ops,
                                        const LoadPlan& plan, const plan::KOrder& ko, int kt, int wave, int wn, int wm,
                                        int r32, int h) {
    // The stage's LDS bases, made opaque in one statement ahead of all its
    // memory operations: the compiler then forms each address at its use
    // (one add) instead of keeping one live register per ring slot and load.
    uint32_t fill_codes = lds_addr(fill) + wave * 4096, fill_scales = lds_addr(fill) + wave * 256, zero = 0;
    asm volatile("" : "+s"(fill_codes), "+s"(fill_scales), "+s"(zero));
    const uint8_t* cur = cur_ + zero;
    const uint8_t* nxt = nxt_ + zero;
    const uint32_t soff = plan::stage_soff(ko, kt + kRing - 1);
    static_for<0, 16>([&](auto n) {
        constexpr int kN = decltype(n)::value;
        mfma_one<0>(acc[kN / 4][kN % 4], f0.w[kN / 4], f0.x[kN % 4], wsc[kN / 4], xsc[kN % 4]);
        if constexpr (ISSUE && kN % 2 == 0) issue_load(kN / 2, fill_codes, fill_scales, ops, plan, soff);
        if constexpr (kN < 8) read_frag<kN>(f1, cur, wn, wm, r32, h, 1);
        __builtin_amdgcn_sched_barrier(0);
    });
    uint32_t wsn[4], xsn[4];
    if (NEXT) ring_barrier<VM>();
    static_for<0, 16>([&](auto n) {
        constexpr int kN = decltype(n)::value;
        // the tile's last K-step may go token block by token block, so the
        // epilogue's first token block can start while the rest finish
        constexpr int kNb = MB_MAJOR ? kN % 4 : kN / 4, kMb = MB_MAJOR ? kN / 4 : kN % 4;
        mfma_one<1>(acc[kNb][kMb], f1.w[kNb], f1.x[kMb], wsc[kNb], xsc[kMb]);
        constexpr int kLate = kN - 6;                          // late loads in slots 6, 7
        if constexpr (ISSUE && kLate >= 0 && kLate < kDmaPerStage - kDmaEarly)
            issue_load(kDmaEarly + kLate, fill_codes, fill_scales, ops, plan, soff);
        if (NEXT) {
            if constexpr (kN < 8)
                read_scale<kN>(wsn, xsn, nxt, wn, wm, r32, h);
            else
                read_frag<kN - 8>(f0, nxt, wn, wm, r32, h, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    if (NEXT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wsc[i] = wsn[i];
            xsc[i] = xsn[i];
        }
    }
}

// Block transform inside the SwiGLU epilogue (KroQuant, "Deep analysis": the
// next layer's input is transformed 32 features at a time, y_b = h_b . T_b).
// Per 32-token x 32-feature block of h it is Y^T = T_b^T . H^T on
// V_MFMA_F32_32X32X16_BF16, two MFMAs over the 32 input features.  The
// contraction order is free, so each lane feeds its own 16 values of h as
// they sit in the accumulator layout (features 8a + 4h + r): MFMA s takes
// hv[8s .. 8s+7] as K slots 8h .. 8h+7, i.e. slot 16s + 8h + e carries
// feature 16s + 8(e/4) + 4h + e%4, and the A operand (lane = output feature
// r32) is gathered from T_b's rows in the same order.  The result has the
// accumulator layout again, ready for the requant.  h is fp32 and the MFMA
// takes bf16, so h is carried as three bf16 parts, hi = bf16(h),
// mid = bf16(h - hi), lo = bf16(h - hi - mid) (each difference is exact in
// fp32): with RNE each part takes the next 8 significant bits of what is
// left, so hi + mid + lo equals h exactly for every h whose residuals stay
// in the normal range (|h| above about 2^-100).  Every bf16 x bf16 product
// is exact in fp32, so y differs from h_b . T_b only by the order of the
// fp32 sums.
__device__ __forceinline__ void load_t_frags(v8s (&tf)[2][2], const GemmArgs& g, int64_t blk0, int r32, int h) {
    // 32-bit element offsets from the scalar base (T is far below 2^31
    // elements), so no per-lane 64-bit address stays live across tiles
    const uint8_t* t8 = reinterpret_cast<const uint8_t*>(g.t);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const uint32_t base = (g.n_t == 1 ? 0u : (uint32_t)(blk0 + p) * 1024u) + (uint32_t)r32;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                tf[p][s][e] = *reinterpret_cast<const short*>(
                    t8 + 2u * (base + (uint32_t)(16 * s + 8 * (e / 4) + 4 * h + e % 4) * 32u));
    }
}

__device__ __forceinline__ void transform_block(float* hv, const v8s (&tf)[2]) {
    v8s hi[2], mid[2], lo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float a = hv[8 * s + e], b = hv[8 * s + e + 1];
            const uint32_t ph = pack_bf16x2(a, b);
            const float ra = a - bf16_bits_to_f32(ph & 0xFFFFu), rb = b - bf16_bits_to_f32(ph >> 16);
            const uint32_t pm = pack_bf16x2(ra, rb);
            const uint32_t pl = pack_bf16x2(ra - bf16_bits_to_f32(pm & 0xFFFFu), rb - bf16_bits_to_f32(pm >> 16));
            hi[s][e] = (short)(ph & 0xFFFFu);
            hi[s][e + 1] = (short)(ph >> 16);
            mid[s][e] = (short)(pm & 0xFFFFu);
            mid[s][e + 1] = (short)(pm >> 16);
            lo[s][e] = (short)(pl & 0xFFFFu);
            lo[s][e + 1] = (short)(pl >> 16);
        }
    // smallest parts first
    v16f y = {};
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[0], lo[0], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[1], lo[1], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[0], mid[0], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[1], mid[1], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[0], hi[0], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[1], hi[1], y, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) hv[i] = y[i];
}

// Epilogue of one tile: per-head RMSNorm / SwiGLU (+ MXFP4 requant) / plain
// cast on the accumulators, then the single store.  `stg` is the LDS ring
// slot left free by the next tile's prefetch: each wave stages its bf16
// rows in its own 8 KiB region of it, and the per-token head sums of a
// 256-wide head (both channel halves) are exchanged through its last 2 KiB.
// acc[nb][mb][i]: channel n0 + wn*128 + nb*32 + 8*(i/4) + 4h + i%4,
//                 token   m0 + wm*128 + mb*32 + r32.
// The next tile's prefetch is issued through the two hooks:
// * plain / RMSNorm: early() runs once this tile's own loads (the norm
//   gains) are issued and before any store, so that every store comes after
//   the prefetch in the in-order VMEM counter and the next tile's first
//   barrier can leave the stores in flight (tile_start_barrier);
// * SwiGLU: after_mb(mb) runs once token block mb is stored (all 256
//   accumulators live at the start leave no registers for the load offsets
//   there; the requant's stores are few).
// MB: token blocks of 32 per wave (4 for a full 256-token tile, 1 for a
// quarter tile of 64 tokens).
// Token block mb's accumulators are read (into VGPRs) from here on, not
// before.  Otherwise the compiler copies all 256 accumulators into VGPRs at
// the start of the epilogue, keeps them there, and has two or three
// temporaries left, so the epilogue's arithmetic runs as one or two
// dependent chains (a single wave issues a dependent chain at well under
// its rate for independent instructions).
template <int MB>
__device__ __forceinline__ void fence_block(v16f (&acc)[4][MB], int mb) {
    asm volatile("" : "+a"(acc[0][mb]), "+a"(acc[1][mb]), "+a"(acc[2][mb]), "+a"(acc[3][mb]));
}

template <int EPI, int OUT, int MB, typename Early, typename AfterMb>
__device__ __forceinline__ void epilogue(v16f (&acc)[4][MB], const GemmArgs& g, int64_t n0, int64_t m0,
                                         uint8_t* stg, int wave, Early early, AfterMb after_mb) {
    const int lane = fresh_lane_id();
    const int wn = wave & 1, wm = wave >> 1;
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t cbase = n0 + wn * 128;
    const int64_t tok0 = m0 + wm * (32 * MB);
    uint8_t* region = stg + wave * kStageOutBytes;
    if (EPI == kEpiNone || EPI == kEpiRmsNorm) {
        float rstd[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) rstd[mb] = 1.f;
        const int64_t head0 = g.head_dim == 256 ? n0 : cbase;
        const bool norm = EPI == kEpiRmsNorm && head0 < g.n_norm;
        // gains through a buffer descriptor sized to n_norm: the loads are
        // unconditional (no branches, so the compiler's VMEM counting stays
        // exact and nothing waits for the prefetch), columns past n_norm read 0
        v4f wv[4][4];
        if (EPI == kEpiRmsNorm) {
            const __amdgpu_buffer_rsrc_t wr =
                buffer_rsrc(reinterpret_cast<const uint8_t*>(g.norm_w), g.norm_w ? g.n_norm * 4 : 0);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const v4u w = __builtin_amdgcn_raw_buffer_load_b128(
                        wr, (int)(cbase + nb * 32 + 8 * a + 4 * h) * 4, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) wv[nb][a][r] = norm ? __uint_as_float(w[r]) : 1.f;
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        early();
        __builtin_amdgcn_sched_barrier(0);
        if (EPI == kEpiRmsNorm) {
            float* red = reinterpret_cast<float*>(stg + kRedOff);   // [2 wn][256 tokens]
            float ss[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
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
                    for (int mb = 0; mb < MB; ++mb) red[wn * kBM + wm * (32 * MB) + mb * 32 + r32] = ss[mb];
                }
                ring_barrier<63>();                       // LDS only: the prefetch stays in flight
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) ss[mb] += red[(1 - wn) * kBM + wm * (32 * MB) + mb * 32 + r32];
                ring_barrier<63>();                       // red overlaps the rows staged next
            }
            // head_dim is 128 or 256: a constant select (an SGPR), not a division whose
            // result would be kept live in a VGPR across the main loop
            const float inv_d = g.head_dim == 256 ? 1.0f / 256.0f : 1.0f / 128.0f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) rstd[mb] = norm ? rsqrtf(ss[mb] * inv_d + g.eps) : 1.f;
        }
        // Columns past n_norm pass through as C * 1 * 1, which is C exactly
        // (rstd and the gains are 1 there), so the bf16 path needs no
        // per-value select (256 fewer VALU per tile); the fp32 path keeps it
        // (without it the compiler spills in one of its instantiations).
        auto vals = [&](int q, int mb, float* v) {
            const int nb = q >> 2, a = q & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[r] = (EPI == kEpiRmsNorm && (OUT == kOutBf16 || norm))
                           ? acc[nb][mb][4 * a + r] * rstd[mb] * wv[nb][a][r]
                           : acc[nb][mb][4 * a + r];
        };
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (OUT == kOutBf16) {
                store_bf16_half<16>(region, [&](int q, float* v) { vals(q, mb, v); }, static_cast<uint16_t*>(g.out),
                                    g.N, tok0 + mb * 32, cbase, g.M, r32, h, lane);
            } else {
                const int64_t tok = tok0 + mb * 32 + r32;
                if (tok < g.M) {
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
    }

    if (EPI == kEpiSwiglu || EPI == kEpiSwigluTransform) {
        // Channel blocks alternate gate / up (interleave group 32): block 2p
        // of the wave holds gate outputs and block 2p+1 the matching up
        // outputs cbase/2 + 32p + 8a + 4h + r.
        const int64_t nh = g.N / 2;
        const int64_t ob0 = cbase / 2;
        v8s tf[2][2];
        if (EPI == kEpiSwigluTransform) load_t_frags(tf, g, ob0 / 32, r32, h);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            // bf16 h: measured 1-3% faster with this token block's reads
            // held back to here (the requant-only path was not: 0-3% slower)
            if (OUT == kOutBf16) fence_block(acc, mb);
            float hv[2][16];                  // [p][4a + r]
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[p][i] = silu_f(acc[2 * p][mb][i]) * acc[2 * p + 1][mb][i];
            if (EPI == kEpiSwigluTransform) {
#pragma unroll
                for (int p = 0; p < 2; ++p) transform_block(hv[p], tf[p]);
            }
            const int64_t tok = tok0 + mb * 32 + r32;
            if (OUT != kOutNone) {
                if (OUT == kOutBf16) {
                    store_bf16_half<8>(region, [&](int q, float* v) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) v[r] = hv[q >> 2][4 * (q & 3) + r];
                    }, static_cast<uint16_t*>(g.out), nh, tok0 + mb * 32, ob0, g.M, r32, h, lane);
                } else if (tok < g.M) {
#pragma unroll
                    for (int p = 0; p < 2; ++p)
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            *reinterpret_cast<v4f*>(static_cast<float*>(g.out) + tok * nh + ob0 + 32 * p + 8 * a +
                                                    4 * h) =
                                (v4f){hv[p][4 * a], hv[p][4 * a + 1], hv[p][4 * a + 2], hv[p][4 * a + 3]};
                }
            }
            if (g.out_codes != nullptr) {
                // Requant of the two 32-output blocks b = ob0/32 + p (p = 0, 1)
                // of token tok.  own[p][j]: this lane's codes of block p,
                // outputs 8a + 4h + r of a = 2j (bytes 0, 1) and a = 2j + 1
                // (bytes 2, 3).  One lane swap of (own[0][j], own[1][j])
                // leaves, in every lane, the h = 0 codes (x) and the h = 1
                // codes (y) of block b + h, so dword a of its 16-byte row is
                // two byte permutes away; lanes h = 0 store both scale bytes
                // (adjacent in the tiled layout, b even) as one u16.
                uint32_t sc[2], own[2][2];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    sc[p] = e8m0_from_amax_bits(max_xor32_u(amax_bits<16>(hv[p])));
                    const float s8 = __uint_as_float(sc[p] << 23);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        uint32_t w = 0u;
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[p][8 * j], hv[p][8 * j + 1], s8, 0);
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[p][8 * j + 2], hv[p][8 * j + 3], s8, 1);
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[p][8 * j + 4], hv[p][8 * j + 5], s8, 2);
                        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, hv[p][8 * j + 6], hv[p][8 * j + 7], s8, 3);
                        own[p][j] = sc[p] == 0xFFu ? 0u : w;     // Inf / NaN block: zero codes
                    }
                }
                v4u st;                                // dword a: outputs 8a .. 8a+7 of block b + h
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const auto xy = __builtin_amdgcn_permlane32_swap(own[0][j], own[1][j], false, false);
                    st[2 * j] = __builtin_amdgcn_perm(xy[1], xy[0], 0x05040100u);
                    st[2 * j + 1] = __builtin_amdgcn_perm(xy[1], xy[0], 0x07060302u);
                }
                if (tok < g.M) {                       // MX_TILED output, ready for the next GEMM
                    // 32-bit offsets: the host keeps both outputs below 2^31 bytes
                    const uint32_t t = (uint32_t)tok, kt = (uint32_t)nh >> 7, blk = (uint32_t)ob0 >> 5;
                    const uint32_t coff = (((t >> 1) * kt + ((blk + h) >> 2)) << 7) + ((t & 1) << 6) + ((blk + h) & 3) * 16;
                    *reinterpret_cast<v4u*>(g.out_codes + coff) = st;
                    if (h == 0)
                        *reinterpret_cast<uint16_t*>(g.out_scales + ((((t >> 5) * kt + (blk >> 2)) << 7) +
                                                                     ((t & 31) << 2) + (blk & 3))) =
                            (uint16_t)(sc[0] | (sc[1] << 8));
                }
            }
            after_mb(mb);
        }
    }
}

// First barrier of a tile after a full-tile plain / RMSNorm epilogue: wait
// for the first prefetched stage only.  VMEM operations issued after it:
// the other prefetched stages (VM0 loads), then the epilogue's stores, 8
// (bf16 rows staged through LDS) or 16 (fp32 rows) per token block; every
// store of a full tile is issued, so VM0 + stores (capped at the counter's
// 63) is at most what follows stage 0.
template <int OUT, int VM0>
__device__ __forceinline__ void tile_start_barrier() {
    constexpr int kStores = 4 * (OUT == kOutBf16 ? 8 : 16);
    ring_barrier<(VM0 + kStores < 63 ? VM0 + kStores : 63)>();
}

// The same after a full-tile SwiGLU epilogue, whose prefetch goes out in two
// pieces: stage 0 after token block 0's stores, stage 1 after block 1's.
// After stage 0 come the stores of blocks 1..3 (3 x per_mb) and stage 1's
// VM0 loads; per_mb = 4 (bf16 h rows) or 8 (fp32) + 2 (code and scale
// stores), as configured.  Each branch's count is at most that.
template <int VM0>
__device__ __forceinline__ void tile_start_barrier_swiglu(int per_mb) {
    if (per_mb >= 10) ring_barrier<VM0 + 30>();
    else if (per_mb >= 8) ring_barrier<VM0 + 24>();
    else if (per_mb >= 6) ring_barrier<VM0 + 18>();
    else if (per_mb >= 4) ring_barrier<VM0 + 12>();
    else if (per_mb >= 2) ring_barrier<VM0 + 6>();
    else ring_barrier<VM0>();
}

// ------------------------------------------------------------ quarter tiles
// When the 256 x 256 tiles leave a partial last round (576 tiles on 256 CUs
// are 2.25 rounds), the tiles of that round are split into quarter tiles of
// 256 channels x 64 tokens, as many as there are workgroups for each of
// them: waves (wn, wm) own 128 channels x 32 tokens (acc[4][1]).  The four
// quarters of a tile run on one XCD, so its weight rows come into one L2.
// Per stage a wave loads 4 weight-code chunks of 16 rows (as in the full
// tile), 16 token rows, its 64 weight-scale rows and all 64 token-scale
// rows: kQDma loads.  It runs once per workgroup at the end,
// where the full tiles' schedule would leave three quarters of the CUs idle.
constexpr int kQDma = 7;

__device__ __forceinline__ void issue_qstage(uint8_t* stage, const Operands& o, const QPlan& p, int kt, int wave,
                                             int lane) {
    const uint32_t soff = (uint32_t)kt * 128u;
    const uint32_t base = opaque_sgpr(lds_addr(stage));
    auto lds = [](uint32_t a) { return (lds_void*)(uintptr_t)a; };
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.wc, lds(base + kWCodesOff + (wave * 4 + j) * 1024), 16, p.w_code[j],
                                                 soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xc, lds(base + kXCodesOff + wave * 1024), 16, p.x_code, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.ws, lds(base + kWScalesOff + wave * 256), 4, p.w_scale, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xs, lds(base + kXScalesOff), 4, p.x_scale, soff, 0, 0);
}

// Load j (0..6, a compile-time constant after inlining) of a quarter stage,
// in issue_qstage's order.
__device__ __forceinline__ void issue_qload(int j, uint32_t base, const Operands& o, const QPlan& p, uint32_t soff,
                                            int wave) {
    auto lds = [](uint32_t a) { return (lds_void*)(uintptr_t)a; };
    if (j < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.wc, lds(base + kWCodesOff + (wave * 4 + j) * 1024), 16, p.w_code[j],
                                                 soff, 0, 0);
    else if (j == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xc, lds(base + kXCodesOff + wave * 1024), 16, p.x_code, soff, 0, 0);
    else if (j == 5)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.ws, lds(base + kWScalesOff + wave * 256), 4, p.w_scale, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o.xs, lds(base + kXScalesOff), 4, p.x_scale, soff, 0, 0);
}

// A quarter stage's operands for one wave: 2 K-steps x (4 weight + 1 token
// fragments) and the scale bytes (a lane's two bytes of the stage, op_sel
// picking one per K-step).
struct QFrags {
    v4i w[2][4], x[2];
    uint32_t wsc[4], xsc;
};

// Read R (0..14) of a quarter stage's operands from ring slot `st`: the 4
// weight scales, the token scale, then per K-step 4 weight and 1 token
// fragments.
template <int R>
__device__ __forceinline__ void read_qfrag(QFrags& f, const uint8_t* st, int wn, int wm, int r32, int h) {
    if constexpr (R < 4) {
        f.wsc[R] = *reinterpret_cast<const uint16_t*>(st + kWScalesOff + (wn * 128 + R * 32 + r32) * kScaleBytes + 2 * h);
    } else if constexpr (R == 4) {
        f.xsc = *reinterpret_cast<const uint16_t*>(st + kXScalesOff + (wm * 32 + r32) * kScaleBytes + 2 * h);
    } else {
        constexpr int kSt = (R - 5) / 5, kI = (R - 5) % 5;
        const int chunk = ((2 * h + kSt) ^ ((r32 >> 2) & 3)) * 16;
        if constexpr (kI < 4)
            f.w[kSt][kI] = *reinterpret_cast<const v4i*>(st + kWCodesOff + (wn * 128 + kI * 32 + r32) * kRowBytes + chunk);
        else
            f.x[kSt] = *reinterpret_cast<const v4i*>(st + kXCodesOff + (wm * 32 + r32) * kRowBytes + chunk);
    }
}

// MFMA I (0..7) of a quarter stage: K-step I / 4, weight fragment I % 4.
template <int I>
__device__ __forceinline__ void q_mfma(v16f (&acc)[4][1], const QFrags& f) {
    mfma_one<I / 4>(acc[I % 4][0], f.w[I / 4][I % 4], f.x[I / 4], f.wsc[I % 4], f.xsc);
}

// Quarter tile (n0, m0: its 256 channels and 64 tokens), software-pipelined
// over the 3-slot ring with three stages in flight: stage kt lives in slot
// kt % 3, and while stage kt is multiplied from registers, the fragments of
// stage kt + 1 are read and the loads of stage kt + 3 go into slot kt % 3,
// whose fragments were read during stage kt - 1.  The 8 MFMAs, 7 loads and
// 15 LDS reads of a stage are interleaved one group per MFMA.  (Measured:
// a quarter tile still takes about 0.7 of a full tile's time for a quarter
// of its work; this schedule took the 4096 x 9216 x 3072 GEMM about 1%
// faster than loads, reads and MFMAs one after the other, and neither
// removing the weight loads nor making every quarter read the same operands
// changed that time much.)  Every stage has the same
// body: near the end of K (and in the prologue when K has fewer than three
// stages) the loads of stages past the last one still go out, but fetch the
// last stage again (plan::qload_stage, a scalar min; the buffer loads'
// scalar offset escapes the hardware's range check, so the stage index
// itself must stay in range) into a slot nobody reads any more, and the
// last stage reads a next stage it never uses, so the loop has no branch
// inside a stage and the barrier count is always one stage of loads.
template <int EPI, int OUT>
__device__ __forceinline__ void quarter_tile(const GemmArgs& g, const Operands& ops, uint8_t* const* slots, int n0,
                                             int m0, int wave) {
    constexpr int D = plan::kQDepth;                   // stages in flight
    const int M = (int)g.M, K = (int)g.K;
    const int kt_count = K / kBK;                      // >= 2
    const int wn = wave & 1, wm = wave >> 1;
    const int lane = fresh_lane_id();
    const int r32 = lane & 31, h = lane >> 5;
    const QPlan qp = make_qplan(M, K, n0, m0, wave, lane);
    ring_barrier<63>();                                // every wave is done with the ring (last epilogue)
    static_for<0, D>([&](auto j) {
        issue_qstage(slots[j()], ops, qp, plan::qload_stage(j(), kt_count), wave, lane);
    });
    ring_barrier<(D - 1) * kQDma>();                   // stage 0 landed
    v16f acc[4][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = (v16f){};
    QFrags fa, fb;
    {
        uint32_t zero = 0;
        asm volatile("" : "+s"(zero));
        const uint8_t* st = slots[0] + zero;
        static_for<0, 15>([&](auto r) { read_qfrag<decltype(r)::value>(fa, st, wn, wm, r32, h); });
    }
    // unrolled by 6 = two ring turns, so that both the slot (kt % 3) and the
    // fragment buffer (kt % 2) are compile-time choices
    for (int kt0 = 0; kt0 < kt_count; kt0 += 6) {
        static_for<0, 6>([&](auto sidx) {
            constexpr int kS = decltype(sidx)::value;
            const int kt = kt0 + kS;
            if (kt < kt_count) {
                QFrags& cur = kS % 2 == 0 ? fa : fb;
                QFrags& nxt = kS % 2 == 0 ? fb : fa;
                // stage kt + 1 landed (stage kt + 2's loads may remain), and
                // every wave has read stage kt's fragments
                ring_barrier<kQDma>();
                uint32_t zero = 0;
                asm volatile("" : "+s"(zero));
                const uint8_t* rd = slots[(kS + 1) % 3] + zero;
                const uint32_t wr = opaque_sgpr(lds_addr(slots[kS % 3]));
                const uint32_t soff = (uint32_t)plan::qload_stage(kt + D, kt_count) * 128u;
                static_for<0, 8>([&](auto i) {
                    constexpr int kI = decltype(i)::value;
                    q_mfma<kI>(acc, cur);
                    if constexpr (kI < 7) issue_qload(kI, wr, ops, qp, soff, wave);
                    read_qfrag<2 * kI>(nxt, rd, wn, wm, r32, h);
                    if constexpr (2 * kI + 1 < 15) read_qfrag<2 * kI + 1>(nxt, rd, wn, wm, r32, h);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
        });
    }
    ring_barrier<0>();                                 // every load landed, every wave done reading
    epilogue<EPI, OUT, 1>(acc, g, n0, m0, slots[0], wave, [] {}, [](int) {});
}

// Persistent kernel: workgroup b runs tiles b, b + G, b + 2G, ... (G = grid
// size, a multiple of 8 so every tile of one workgroup maps to its own XCD).
// The first NS - 1 K stages of the next tile load while the current tile's
// epilogue runs, one stage after each of its first token blocks is stored.
// NS: ring depth (kRing); PEEL: (K/128 - NS + 1) % NS, the stages run before
// the unrolled loop.
template <int EPI, int OUT, int NS, int PEEL>
__global__ __launch_bounds__(256, 1) void gemm_fp4_kernel(GemmArgs g) {
    static_assert(NS >= 2 && NS <= kRing && PEEL <= NS, "ring shape");
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t ring1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t ring2[NS > 2 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t ring3[NS > 3 ? kStageBytes : 16];

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wn = wave & 1;              // channel half of the workgroup tile (128 channels)
    const int wm = wave >> 1;             // token half (128 tokens)
    const int M = (int)g.M, K = (int)g.K;    // M * K / 2 < 2^31 (checked by the host)
    const int tiles_n = (int)(g.N / kBN);
    const int tiles_m = (M + kBM - 1) / kBM;
    const int n_tiles = tiles_n * tiles_m;
    const int kt_count = K / kBK;            // >= NS - 1 (the host requires K >= 256)
    const Operands ops = make_operands(g);

    // Stage j lives in ring slot (j + OFF) % NS.  The first PEEL stages run
    // before the unrolled loop, so the loop always starts on slot 0 and the
    // last NS - 1 stages sit in slots 0 .. NS - 2: every slot index is a
    // compile-time constant, and slot OFF - 1 (mod NS) is the one the next
    // tile's prefetch leaves free for the epilogue.
    constexpr int D = NS - 1;                          // prefetch distance (stages)
    constexpr int OFF = (NS - PEEL) % NS;
    // loads that may still be in flight at a barrier: in the K loop, those of
    // the D - 1 later stages issued before it; at a tile's start, the whole
    // prefetched stages after stage 0
    constexpr int kVmSteady = (D - 1) * kDmaEarly;
    constexpr int kVmPrologue = (D - 1) * kDmaPerStage;
    uint8_t* const slots[4] = {ring0, ring1, ring2, ring3};
    uint8_t* const stg = slots[(OFF + D) % NS];
    const int n_issue = kt_count - D;
    constexpr bool kEarly = EPI == kEpiNone || EPI == kEpiRmsNorm;

    // A partial last round of full tiles runs as quarter tiles instead (plain
    // and RMSNorm epilogues; the round's tile count a multiple of the 8 XCDs):
    // virtual tiles [0, n_full) are full, [n_full, n_virtual) quarters.
    int n_full = n_tiles, n_virtual = n_tiles;
    if constexpr (kEarly) {
        const int G = (int)gridDim.x, rem = n_tiles % G;
        if (rem != 0 && (rem & 7) == 0 && (G & 7) == 0) {
            n_full = n_tiles - rem;
            n_virtual = n_full + 4 * rem;
        }
    }

    int v = blockIdx.x;
    bool relaxed = false;
    int tm, tn;
    int nth = 0;                                       // tiles this workgroup has started
    plan::KOrder ko = plan::k_order(nth, kt_count);
    tile_of(v, n_tiles, tiles_n, tiles_m, tm, tn);
    {
        const LoadPlan plan = make_plan(M, K, tn * kBN, tm * kBM, wave, fresh_lane_id());
        static_for<0, D>([&](auto j) {
            issue_stage_at(slots[(j() + OFF) % NS], ops, plan, plan::stage_soff(ko, j()), wave);
        });
    }

    for (;;) {
        const int n0 = tn * kBN;
        const int m0 = tm * kBM;
        const int lane = fresh_lane_id();
        const int r32 = lane & 31;
        const int h = lane >> 5;
        const LoadPlan plan = make_plan(M, K, n0, m0, wave, lane);
        v16f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

        if (relaxed) {                                 // stage 0 landed; stores may still drain
            if constexpr (kEarly)
                tile_start_barrier<OUT, kVmPrologue>();
            else
                // (without `out` the requant output is always set)
                tile_start_barrier_swiglu<kVmPrologue>(
                    OUT == kOutNone ? 2
                                    : __builtin_amdgcn_readfirstlane((OUT == kOutBf16 ? 4 : 8) +
                                                                     (g.out_codes == nullptr ? 0 : 2)));
        } else {
            ring_barrier<kVmPrologue>();
        }
        Frags f0, f1;
        uint32_t wsc[4], xsc[4];
        read_scales(wsc, xsc, slots[OFF % NS], wn, wm, r32, h);
        read_frags(f0, slots[OFF % NS], wn, wm, r32, h, 0);

        // stages 0 .. PEEL-1 (each issues the loads of stage j + D)
        static_for<0, PEEL>([&](auto j) {
            k_stage<true, true, kVmSteady>(acc, f0, f1, wsc, xsc, slots[(j() + OFF) % NS],
                                           slots[(j() + OFF + 1) % NS], slots[(j() + OFF + D) % NS], ops, plan, ko, j(),
                                           wave, wn, wm, r32, h);
        });
        // stages PEEL .. kt_count - NS, NS at a time, on slots 0 .. NS-1
        for (int kt = PEEL; kt < n_issue; kt += NS) {
            static_for<0, NS>([&](auto s) {
                k_stage<true, true, kVmSteady>(acc, f0, f1, wsc, xsc, slots[s()], slots[(s() + 1) % NS],
                                               slots[(s() + D) % NS], ops, plan, ko, kt + s(), wave, wn, wm, r32, h);
            });
        }
        // the last D stages: no more loads; stage n_issue + i waits for the
        // D - 2 - i stages still behind the next one
        static_for<0, D>([&](auto i) {
            constexpr int kI = decltype(i)::value;
            constexpr int kVm = kI < D - 1 ? (D - 2 - kI) * kDmaPerStage : 0;
            k_stage<false, (kI < D - 1), kVm, (kI == D - 1)>(acc, f0, f1, wsc, xsc, slots[kI], slots[(kI + 1) % NS],
                                                             slots[0], ops, plan, ko, n_issue + kI, wave, wn, wm,
                                                             r32, h);
        });
        // All 16 accumulator blocks pass through one empty asm statement:
        // every last MFMA issues before the epilogue reads any accumulator.
        // Otherwise the scheduler puts reads of a just-written block between
        // the last MFMAs, and each such read holds the wave's issue until
        // that MFMA has finished, so the next MFMA waits too.  With the last
        // K-step ordered by token block, block 0's results are ready first.
        asm volatile(""
                     : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                       "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
                       "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
                       "+a"(acc[3][3]));
        ring_barrier<63>();                            // every wave is done reading the ring

        const int vn = v + (int)gridDim.x;
        const bool more = vn < n_full;                 // the next tile is a full one
        if (more) tile_of(vn, n_tiles, tiles_n, tiles_m, tm, tn);
        ko = plan::k_order(++nth, kt_count);           // the next tile's K order
        // finish this tile; the next full tile's first stages load meanwhile
        // (their load offsets are formed there rather than kept live through
        // the epilogue)
        epilogue<EPI, OUT, 4>(
            acc, g, n0, m0, stg, wave,
            [&]() {
                if (kEarly && more) {
                    const LoadPlan pl = make_plan(M, K, tn * kBN, tm * kBM, wave, fresh_lane_id());
                    static_for<0, D>([&](auto j) {
                        issue_stage_at(slots[(j() + OFF) % NS], ops, pl, plan::stage_soff(ko, j()), wave);
                    });
                }
            },
            [&](int mb) {
                if (!kEarly && more && mb < D)
                    issue_stage_at(slots[(mb + OFF) % NS], ops,
                                   make_plan(M, K, tn * kBN, tm * kBM, wave, fresh_lane_id()),
                                   plan::stage_soff(ko, mb), wave);
            });
        if (!more) {
            if constexpr (kEarly) v = vn;              // on to the quarter tiles
            break;
        }
        // after a full tile every store of the epilogue was issued (the
        // plain / RMSNorm ones all after the prefetch)
        relaxed = __builtin_amdgcn_readfirstlane((int)(m0 + kBM <= M)) != 0;   // uniform: keep it scalar
        v = vn;
    }
    // quarter tiles: q = v - n_full -> XCD q % 8, quarter (q / 8) % 4 of the
    // partial round's tile n_full + (q / 32) * 8 + q % 8 (workgroup ids, and
    // so q, are congruent to their XCD mod 8: a tile's quarters share one)
    if constexpr (kEarly) {
        for (; v < n_virtual; v += (int)gridDim.x) {
            const int q = v - n_full;
            int ptm, ptn;
            tile_of(n_full + ((q >> 5) << 3) + (q & 7), n_tiles, tiles_n, tiles_m, ptm, ptn);
            quarter_tile<EPI, OUT>(g, ops, slots, ptn * kBN, ptm * kBM + ((q >> 3) & 3) * 64, wave);
        }
    }
}

template <int EPI, int OUT, int NS>
void launch_peel(const GemmArgs& g, int peel, dim3 grid, hipStream_t stream) {
    static_for_host<0, NS + 1>([&](auto p) {
        constexpr int kPeel = decltype(p)::value;
        if (peel == kPeel)
            hipLaunchKernelGGL((gemm_fp4_kernel<EPI, OUT, NS, kPeel>), grid, dim3(256), 0, stream, g);
    });
}

// A kRing-deep ring needs at least kRing - 1 K stages: K >= 256 gives two.
template <int EPI, int OUT>
void launch_ring(const GemmArgs& g, dim3 grid, hipStream_t stream) {
    static_assert(kRing - 1 <= kGemmKMin / kBK && kGemmKMultiple % kBK == 0, "ring deeper than the shortest K");
    const int kt_count = (int)(g.K / kBK);
    // With no stage to peel (K/128 - 2 a multiple of 3) the compiler copies
    // every accumulator on entering and leaving the unrolled loop (measured:
    // the main loop ran 25% slower); peeling one whole ring turn instead
    // keeps them in place.  Needs kRing stages ahead of the loop.
    int peel = (kt_count - (kRing - 1)) % kRing;
    if (peel == 0 && kt_count - (kRing - 1) >= kRing) peel = kRing;
    launch_peel<EPI, OUT, kRing>(g, peel, grid, stream);
}

// `out` NULL (only the SwiGLU epilogues allow it: their requant output is
// set then), bf16 or fp32.
template <int EPI>
void launch_epi(const GemmArgs& g, bool out_bf16, dim3 grid, hipStream_t stream) {
    if constexpr (EPI == kEpiSwiglu || EPI == kEpiSwigluTransform) {
        if (g.out == nullptr) {
            launch_ring<EPI, kOutNone>(g, grid, stream);
            return;
        }
    }
    if (out_bf16) {
        launch_ring<EPI, kOutBf16>(g, grid, stream);
    } else {
        launch_ring<EPI, kOutF32>(g, grid, stream);
    }
}

// Compute units of the current device (cached per device).
// CU count per device, cached (atomically: host threads may launch at once;
// a race only makes two of them query the same value).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_gemm(const GemmArgs& g, int epi, bool out_bf16, hipStream_t stream) {
    const int64_t tiles = (g.N / kBN) * ((g.M + kBM - 1) / kBM);
    // one workgroup per CU, a multiple of 8 (the XCD count) when persistent
    const int64_t cus = device_cus();
    const int64_t wgs = tiles <= cus ? tiles : (cus >= 8 ? cus & ~int64_t(7) : cus);
    const dim3 grid((unsigned)wgs);
    switch (epi) {
        case kEpiNone: launch_epi<kEpiNone>(g, out_bf16, grid, stream); break;
        case kEpiRmsNorm: launch_epi<kEpiRmsNorm>(g, out_bf16, grid, stream); break;
        case kEpiSwiglu: launch_epi<kEpiSwiglu>(g, out_bf16, grid, stream); break;
        default: launch_epi<kEpiSwigluTransform>(g, out_bf16, grid, stream); break;
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

hipError_t launch_gemm_swiglu_transform(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                                        const uint8_t* bc, const uint8_t* bs, const uint16_t* t, int64_t n_t,
                                        void* out, bool out_bf16, uint8_t* out_codes, uint8_t* out_scales,
                                        hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out;
    g.out_codes = out_codes; g.out_scales = out_scales;
    g.t = t; g.n_t = n_t;
    return launch_gemm(g, kEpiSwigluTransform, out_bf16, stream);
}

}  // namespace fp4dit
