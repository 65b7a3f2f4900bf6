// Fused MXFP4 GEMM + epilogue for gfx950 (CDNA4).
//
// fal, epilogue-fusion section: the GEMM forms A . B tile by tile with the
// accumulators on chip, and the small ops that follow it (per-head RMSNorm
// on the attention path, gated SiLU in the FFN, the output cast) run on those
// accumulators before the single store, so the GEMM output never makes an
// extra HBM round trip.  KroQuant, "Deep analysis": both operands are MXFP4.
//
// Design (MI355X-first; the Blackwell tiling on the fal page is prior art):
// * Contraction on V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands: it
//   reaches the FP4 matrix rate, while the 16x16x128 shape only reaches half
//   of it on this chip.  Its scale operand carries one e8m0 byte per lane,
//   which is exactly one MX block (lane l holds row l%32, 32 K-elements).
// * The GEMM is computed transposed, D = W . X^T: the weight rows (output
//   channels) are the MFMA "A" operand and the tokens the "B" operand, so a
//   lane's 16 accumulators of a 32x32 block are 4 runs of 4 consecutive
//   channels of one token.  Per-head sums then need one cross-lane step
//   (lane l and l^32) and stores are 8/16-byte vectors.
// * Workgroup tile 256 channels x 256 tokens, 4 waves of 128 x 128 (256 fp32
//   accumulators per lane), K staged 256 at a time through LDS, double
//   buffered (2 x 68 KiB).  Global -> LDS uses the direct-to-LDS
//   global_load_lds_dwordx4 (no VGPR staging); a row's 16-byte chunks are
//   XOR-swizzled with the row index so the fragment reads (ds_read_b128,
//   8 rows per 128 bytes) are free of bank conflicts.
// * K is permuted inside a stage: in K-step s lane group h (= lane / 32)
//   takes MX block 4h + s, so a lane's four scale bytes of a stage are
//   adjacent, one ds_read_b32 fetches them and op_sel picks the byte.  Both
//   operands use the same permutation, so the sum over K is unchanged.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp4dit {
namespace {

constexpr int kBM = 256;              // tokens per workgroup
constexpr int kBN = 256;              // channels per workgroup
constexpr int kBK = 256;              // K elements per LDS stage
constexpr int kRowBytes = kBK / 2;    // 128 bytes of codes per row per stage
constexpr int kScaleBytes = kBK / 32; // 8 scale bytes per row per stage
constexpr int kWCodesOff = 0;
constexpr int kXCodesOff = kWCodesOff + kBN * kRowBytes;        // 32 KiB
constexpr int kWScalesOff = kXCodesOff + kBM * kRowBytes;       // 64 KiB
constexpr int kXScalesOff = kWScalesOff + kBN * kScaleBytes;    // +2 KiB
constexpr int kStageBytes = kXScalesOff + kBM * kScaleBytes;    // 68 KiB
constexpr int kLdsBytes = 2 * kStageBytes;                      // 136 KiB

enum EpiKind { kEpiNone = 0, kEpiRmsNorm = 1, kEpiSwiglu = 2 };

struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    void* out;
    int out_bf16;
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

// Per-lane state of the direct-to-LDS loads: 32-bit byte offsets from the
// operand base, fixed for the whole K loop (the K stage advances the
// wave-uniform base instead, so the loads use the SGPR-base addressing form).
struct LoadPlan {
    uint32_t w_code[8], x_code[8];    // 8 groups of 8 rows x 128 B per operand
    uint32_t w_scale[2], x_scale[2];  // 2 groups of 32 rows x 8 B per operand
};

__device__ __forceinline__ LoadPlan make_plan(const GemmArgs& g, int64_t n0, int64_t m0, int wave, int lane) {
    LoadPlan p;
    const uint32_t kcb = (uint32_t)(g.K / 2);
    const uint32_t ksb = (uint32_t)(g.K / 32);
    const int rin = lane >> 3;             // row within an 8-row group
    const int lchunk = (lane & 7) ^ rin;   // logical chunk written to physical chunk lane & 7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = (wave * 8 + j) * 8 + rin;
        int64_t xr = m0 + row;
        xr = xr < g.M ? xr : g.M - 1;     // ragged token tile: clamp, never stored
        p.w_code[j] = (uint32_t)(n0 + row) * kcb + lchunk * 16;
        p.x_code[j] = (uint32_t)xr * kcb + lchunk * 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = (wave * 2 + j) * 32 + (lane >> 1);
        int64_t xr = m0 + row;
        xr = xr < g.M ? xr : g.M - 1;
        p.w_scale[j] = (uint32_t)(n0 + row) * ksb + (lane & 1) * 4;
        p.x_scale[j] = (uint32_t)xr * ksb + (lane & 1) * 4;
    }
    return p;
}

// Enqueue the direct-to-LDS loads of K stage kt into `stage`.
__device__ __forceinline__ void issue_stage(uint8_t* stage, const GemmArgs& g, const LoadPlan& p,
                                            int kt, int wave) {
    const uint8_t* wc = g.b_codes + (int64_t)kt * kRowBytes;
    const uint8_t* xc = g.a_codes + (int64_t)kt * kRowBytes;
    const uint8_t* ws = g.b_scales + (int64_t)kt * kScaleBytes;
    const uint8_t* xs = g.a_scales + (int64_t)kt * kScaleBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int grp = wave * 8 + j;
        __builtin_amdgcn_global_load_lds(wc + p.w_code[j], (lds_void*)(stage + kWCodesOff + grp * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(xc + p.x_code[j], (lds_void*)(stage + kXCodesOff + grp * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int grp = wave * 2 + j;
        __builtin_amdgcn_global_load_lds(ws + p.w_scale[j], (lds_void*)(stage + kWScalesOff + grp * 256), 4, 0, 0);
        __builtin_amdgcn_global_load_lds(xs + p.x_scale[j], (lds_void*)(stage + kXScalesOff + grp * 256), 4, 0, 0);
    }
}

struct Frags {
    v4i w[4], x[4];
};

// Fragment reads of K-step s: lane group h takes MX block 4h + s of the stage.
__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* stage, int wn, int wm, int r32, int h,
                                           int swz, int s) {
    const int chunk = ((4 * h + s) ^ swz) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.w[i] = *reinterpret_cast<const v4i*>(stage + kWCodesOff + (wn * 128 + i * 32 + r32) * kRowBytes + chunk);
        f.x[i] = *reinterpret_cast<const v4i*>(stage + kXCodesOff + (wm * 128 + i * 32 + r32) * kRowBytes + chunk);
    }
}

__device__ __forceinline__ void read_scales(uint32_t* wsc, uint32_t* xsc, const uint8_t* stage, int wn, int wm,
                                            int r32, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wsc[i] = *reinterpret_cast<const uint32_t*>(stage + kWScalesOff + (wn * 128 + i * 32 + r32) * kScaleBytes + h * 4);
        xsc[i] = *reinterpret_cast<const uint32_t*>(stage + kXScalesOff + (wm * 128 + i * 32 + r32) * kScaleBytes + h * 4);
    }
}

template <int S>
__device__ __forceinline__ void mfma_step(v16f (&acc)[4][4], const Frags& f, const uint32_t* wsc, const uint32_t* xsc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v8i a = {f.w[i][0], f.w[i][1], f.w[i][2], f.w[i][3], 0, 0, 0, 0};
            const v8i b = {f.x[j][0], f.x[j][1], f.x[j][2], f.x[j][3], 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 4, 4, S, (int)wsc[i],
                                                                        S, (int)xsc[j]);
        }
}

// Scheduling of one K-step: its 16 MFMAs interleaved with the 8 fragment
// reads of the next K-step (one read, then two MFMAs), and in the first step
// of a stage also with the 20 direct-to-LDS loads of the following stage.
// Masks: 0x008 MFMA, 0x010 VMEM, 0x100 DS read.
__device__ __forceinline__ void interleave_reads_mfma() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void interleave_loads_reads_mfma() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x010, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void interleave_scales_reads_mfma() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Map the linear workgroup id to a (token tile, channel tile).  Workgroups
// are dispatched round-robin over the 8 XCDs; consecutive remapped ids land
// on one XCD and walk a band of 4 token tiles across the channel tiles, so
// the workgroups an XCD runs together share operand rows in its L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t nwg, int64_t tiles_n, int64_t tiles_m,
                                        int64_t& tm, int64_t& tn) {
    int64_t b = bid;
    if ((nwg & 7) == 0) b = (bid & 7) * (nwg >> 3) + (bid >> 3);
    constexpr int64_t kGroupM = 4;
    const int64_t per_group = kGroupM * tiles_n;
    const int64_t group = b / per_group;
    const int64_t first = group * kGroupM;
    const int64_t gm = (tiles_m - first) < kGroupM ? (tiles_m - first) : kGroupM;
    const int64_t in = b - group * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_fp4_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;              // channel half of the workgroup tile
    const int wm = wave >> 1;             // token half
    const int64_t tiles_n = g.N / kBN;
    const int64_t tiles_m = (g.M + kBM - 1) / kBM;
    int64_t tm, tn;
    tile_of(blockIdx.x, (int64_t)gridDim.x, tiles_n, tiles_m, tm, tn);
    const int64_t n0 = tn * kBN;
    const int64_t m0 = tm * kBM;
    const int kt_count = (int)(g.K / kBK);

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

    const int r32 = lane & 31;
    const int h = lane >> 5;
    const int swz = lane & 7;             // row & 7 of every fragment row this lane reads

    const LoadPlan plan = make_plan(g, n0, m0, wave, lane);
    issue_stage(smem, g, plan, 0, wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    Frags f0, f1;
    uint32_t wsc[4], xsc[4], wsn[4], xsn[4];
    read_scales(wsc, xsc, smem, wn, wm, r32, h);
    read_frags(f0, smem, wn, wm, r32, h, swz, 0);

    // Steady state: stage kt is computed while stage kt+1 streams in.  The
    // loop body has no branches (the last stage is peeled below) so the
    // compiler keeps the MFMAs interleaved with the fragment reads.
    for (int kt = 0; kt < kt_count - 1; ++kt) {
        const uint8_t* cur = smem + (kt & 1) * kStageBytes;
        uint8_t* nxt = smem + ((kt + 1) & 1) * kStageBytes;
        issue_stage(nxt, g, plan, kt + 1, wave);
        read_frags(f1, cur, wn, wm, r32, h, swz, 1);
        mfma_step<0>(acc, f0, wsc, xsc);
        interleave_loads_reads_mfma();
        read_frags(f0, cur, wn, wm, r32, h, swz, 2);
        mfma_step<1>(acc, f1, wsc, xsc);
        interleave_reads_mfma();
        read_frags(f1, cur, wn, wm, r32, h, swz, 3);
        mfma_step<2>(acc, f0, wsc, xsc);
        interleave_reads_mfma();
        // Every wave has its stage-kt fragments in registers and its
        // stage-kt+1 loads landed: after this barrier the next stage may be
        // read and this one overwritten.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        read_scales(wsn, xsn, nxt, wn, wm, r32, h);
        read_frags(f0, nxt, wn, wm, r32, h, swz, 0);
        mfma_step<3>(acc, f1, wsc, xsc);
        interleave_scales_reads_mfma();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wsc[i] = wsn[i];
            xsc[i] = xsn[i];
        }
    }
    {
        const uint8_t* cur = smem + ((kt_count - 1) & 1) * kStageBytes;
        read_frags(f1, cur, wn, wm, r32, h, swz, 1);
        mfma_step<0>(acc, f0, wsc, xsc);
        interleave_reads_mfma();
        read_frags(f0, cur, wn, wm, r32, h, swz, 2);
        mfma_step<1>(acc, f1, wsc, xsc);
        interleave_reads_mfma();
        read_frags(f1, cur, wn, wm, r32, h, swz, 3);
        mfma_step<2>(acc, f0, wsc, xsc);
        interleave_reads_mfma();
        mfma_step<3>(acc, f1, wsc, xsc);
    }
    __syncthreads();                      // the epilogue may reuse the LDS

    // ------------------------------------------------------------ epilogue --
    // acc[nb][mb][i]: channel n0 + wn*128 + nb*32 + 8*(i/4) + 4h + i%4,
    //                 token   m0 + wm*128 + mb*32 + r32.
    const int64_t cbase = n0 + wn * 128;
    if (EPI == kEpiNone || EPI == kEpiRmsNorm) {
        float rstd[4] = {1.f, 1.f, 1.f, 1.f};
        bool norm = false;
        if (EPI == kEpiRmsNorm) {
            float* red = reinterpret_cast<float*>(smem);  // [2 wn][256 tokens]
            float ss[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
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
                    for (int mb = 0; mb < 4; ++mb) red[wn * 256 + wm * 128 + mb * 32 + r32] = ss[mb];
                }
                __syncthreads();
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) ss[mb] += red[(1 - wn) * 256 + wm * 128 + mb * 32 + r32];
            }
            const int64_t head0 = g.head_dim == 256 ? n0 : cbase;
            norm = head0 < g.n_norm;
            const float inv_d = 1.0f / (float)g.head_dim;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) rstd[mb] = rsqrtf(ss[mb] * inv_d + g.eps);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int64_t ch = cbase + nb * 32 + 8 * a + 4 * h;
                v4f wv = {1.f, 1.f, 1.f, 1.f};
                if (EPI == kEpiRmsNorm && norm) wv = *reinterpret_cast<const v4f*>(g.norm_w + ch);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const int64_t tok = m0 + wm * 128 + mb * 32 + r32;
                    if (tok >= g.M) continue;
                    const v16f& c = acc[nb][mb];
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = (EPI == kEpiRmsNorm && norm) ? c[4 * a + r] * rstd[mb] * wv[r] : c[4 * a + r];
                    if (OUT_BF16) {
                        v2u o;
                        o[0] = pack_bf16x2(v[0], v[1]);
                        o[1] = pack_bf16x2(v[2], v[3]);
                        *reinterpret_cast<v2u*>(static_cast<uint16_t*>(g.out) + tok * g.N + ch) = o;
                    } else {
                        *reinterpret_cast<v4f*>(static_cast<float*>(g.out) + tok * g.N + ch) =
                            (v4f){v[0], v[1], v[2], v[3]};
                    }
                }
            }
    }

    if (EPI == kEpiSwiglu) {
        // Channel blocks alternate gate / up (interleave group 32): block
        // 2q holds gate outputs and block 2q+1 the matching up outputs
        // cbase/2 + 32q + 8a + 4h + r.
        const int64_t nh = g.N / 2;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int64_t tok = m0 + wm * 128 + mb * 32 + r32;
            const bool live = tok < g.M;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float hv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[i] = silu_f(acc[2 * q][mb][i]) * acc[2 * q + 1][mb][i];
                const int64_t ob = cbase / 2 + 32 * q;   // first output of this 32-block
                if (g.out != nullptr && live) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int64_t oc = ob + 8 * a + 4 * h;
                        if (OUT_BF16) {
                            v2u v;
                            v[0] = pack_bf16x2(hv[4 * a + 0], hv[4 * a + 1]);
                            v[1] = pack_bf16x2(hv[4 * a + 2], hv[4 * a + 3]);
                            *reinterpret_cast<v2u*>(static_cast<uint16_t*>(g.out) + tok * nh + oc) = v;
                        } else {
                            const v4f v = {hv[4 * a + 0], hv[4 * a + 1], hv[4 * a + 2], hv[4 * a + 3]};
                            *reinterpret_cast<v4f*>(static_cast<float*>(g.out) + tok * nh + oc) = v;
                        }
                    }
                }
                if (g.out_codes != nullptr) {
                    uint32_t hb[16];
                    uint32_t amax = 0u;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        hb[i] = __float_as_uint(hv[i]);
                        const uint32_t a = hb[i] & 0x7FFFFFFFu;
                        amax = a > amax ? a : amax;
                    }
                    amax = max_xor32_u(amax);
                    const uint32_t sc = e8m0_from_amax_bits(amax);
                    uint32_t c16[4];                  // codes of outputs 8a+4h .. +3
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        uint32_t w = 0u;
#pragma unroll
                        for (int r = 0; r < 4; ++r) w |= e2m1_code(hb[4 * a + r], sc) << (4 * r);
                        c16[a] = sc == 0xFFu ? 0u : w;
                    }
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
                    if (live) {
                        const int64_t blk = ob / 32;
                        *reinterpret_cast<v2u*>(g.out_codes + tok * (nh / 2) + blk * 16 + h * 8) = st;
                        if (h == 0) g.out_scales[tok * (nh / 32) + blk] = (uint8_t)sc;
                    }
                }
            }
        }
    }
}

template <int EPI>
void launch_epi(const GemmArgs& g, dim3 grid, hipStream_t stream) {
    if (g.out_bf16) {
        hipLaunchKernelGGL((gemm_fp4_kernel<EPI, true>), grid, dim3(256), 0, stream, g);
    } else {
        hipLaunchKernelGGL((gemm_fp4_kernel<EPI, false>), grid, dim3(256), 0, stream, g);
    }
}

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t stream) {
    const int64_t tiles = (g.N / kBN) * ((g.M + kBM - 1) / kBM);
    const dim3 grid((unsigned)tiles);
    switch (epi) {
        case kEpiNone: launch_epi<kEpiNone>(g, grid, stream); break;
        case kEpiRmsNorm: launch_epi<kEpiRmsNorm>(g, grid, stream); break;
        default: launch_epi<kEpiSwiglu>(g, grid, stream); break;
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
    g.out = out; g.out_bf16 = out_bf16 ? 1 : 0;
    return launch_gemm(g, kEpiNone, stream);
}

hipError_t launch_gemm_rmsnorm(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                               const uint8_t* bc, const uint8_t* bs, int head_dim, int64_t n_norm,
                               const float* norm_w, float eps, void* out, bool out_bf16,
                               hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out; g.out_bf16 = out_bf16 ? 1 : 0;
    g.head_dim = head_dim; g.n_norm = n_norm; g.norm_w = norm_w; g.eps = eps;
    return launch_gemm(g, kEpiRmsNorm, stream);
}

hipError_t launch_gemm_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                              const uint8_t* bc, const uint8_t* bs, void* out, bool out_bf16,
                              uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a_codes = ac; g.a_scales = as; g.b_codes = bc; g.b_scales = bs;
    g.out = out; g.out_bf16 = out_bf16 ? 1 : 0;
    g.out_codes = out_codes; g.out_scales = out_scales;
    return launch_gemm(g, kEpiSwiglu, stream);
}

}  // namespace fp4dit
