// Host-side bounds walk of the fused GEMM's direct-to-LDS operand loads,
// built from the kernel's own load-plan code (csrc/gemm_plan.hpp).
//
// For each GEMM shape M N K given on the command line, every 256 x 256 tile
// (in both of its K orders) and every 256 x 64 quarter of it, every wave and
// lane, and every K stage a load is issued for, the byte range a load reads must lie inside the
// operand buffer (the tiled buffer size, which is also the record count of
// the kernel's buffer descriptor).  The scalar stage offset of these buffer
// loads is not range-checked by the hardware, so this is the only guard.
//
// Usage: plan_check [--unclamped] M N K [M N K ...]
//   --unclamped  model the quarter loop without its stage clamp (the loads of
//                positions past the last stage fetch those stages): used by
//                the test to show that the walk catches that mistake.
// Prints "ok <loads checked>" per shape, or the first out-of-range load and
// exits 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gemm_plan.hpp"

using namespace fp4dit::plan;

static long long g_checked = 0;

static bool in_range(const char* what, int64_t off, int width, int64_t bytes, int tile_n, int tile_m, int wave,
                     int lane, int stage) {
    ++g_checked;
    if (off < 0 || off + width > bytes) {
        std::printf("out of range: %s offset %lld + %d > %lld bytes (tile n0=%d m0=%d wave %d lane %d stage %d)\n",
                    what, (long long)off, width, (long long)bytes, tile_n, tile_m, wave, lane, stage);
        return false;
    }
    return true;
}

// Each K order visits every stage exactly once, on 128-byte stage boundaries.
static bool check_orders(int kt_count) {
    for (int nth = 0; nth < 2; ++nth) {
        const KOrder ko = k_order(nth, kt_count);
        std::vector<int> seen(kt_count, 0);
        for (int i = 0; i < kt_count; ++i) {
            const int64_t so = (int64_t)(int32_t)stage_soff(ko, i);
            if (so < 0 || so % kBK != 0 || so / kBK >= kt_count || seen[so / kBK]++) {
                std::printf("K order %d: position %d gives offset %lld (%d stages)\n", nth, i, (long long)so, kt_count);
                return false;
            }
        }
    }
    return true;
}

static bool check_shape(int M, int N, int K, bool unclamped) {
    const int kt_count = K / kBK;
    if (!check_orders(kt_count)) return false;
    const int64_t wc = code_bytes(N, K), xc = code_bytes(M, K), ws = scale_bytes(N, K), xs = scale_bytes(M, K);
    const int tiles_n = N / 256, tiles_m = (M + 255) / 256;
    // the extreme stages suffice for the large shapes (offsets grow with the stage)
    const bool all_stages = (long long)tiles_n * tiles_m * kt_count <= 4096;
    for (int tn = 0; tn < tiles_n; ++tn)
        for (int tm = 0; tm < tiles_m; ++tm) {
            const int n0 = tn * 256, m0 = tm * 256;
            for (int wave = 0; wave < 4; ++wave)
                for (int lane = 0; lane < 64; ++lane) {
                    // full tile: K positions 0 .. kt_count - 1 (the prefetch of a
                    // tile's first stages included), in both K orders (a
                    // workgroup's even and odd tiles)
                    const LoadPlan p = make_plan(M, K, n0, m0, wave, lane);
                    for (int nth = 0; nth < 2; ++nth) {
                        const KOrder ko = k_order(nth, kt_count);
                        for (int i = 0; i < kt_count; ++i) {
                            if (!all_stages && i != 0 && i != kt_count - 1) continue;
                            const int64_t so = (int64_t)(int32_t)stage_soff(ko, i);
                            const int kt = (int)(so / kBK);
                            for (int j = 0; j < 4; ++j) {
                                if (!in_range("weight codes", p.w_code[j] + so, 16, wc, n0, m0, wave, lane, kt)) return false;
                                if (!in_range("token codes", p.x_code[j] + so, 16, xc, n0, m0, wave, lane, kt)) return false;
                            }
                            if (!in_range("weight scales", p.w_scale + so, 4, ws, n0, m0, wave, lane, kt)) return false;
                            if (!in_range("token scales", p.x_scale + so, 4, xs, n0, m0, wave, lane, kt)) return false;
                        }
                    }
                    // quarter tiles: load positions 0 .. kt_count + kQDepth - 1
                    // (the prologue's kQDepth stages, then stage kt + kQDepth
                    // during stage kt)
                    for (int q = 0; q < 4; ++q) {
                        const int qm0 = m0 + q * 64;
                        const QPlan qp = make_qplan(M, K, n0, qm0, wave, lane);
                        for (int s = 0; s < kt_count + kQDepth; ++s) {
                            const int st = unclamped ? s : qload_stage(s, kt_count);
                            if (!unclamped && (st < 0 || st >= kt_count)) {
                                std::printf("stage %d of position %d outside [0, %d)\n", st, s, kt_count);
                                return false;
                            }
                            if (!all_stages && s != 0 && s < kt_count + kQDepth - 1) continue;
                            const int64_t so = (int64_t)st * kBK;
                            for (int j = 0; j < 4; ++j)
                                if (!in_range("quarter weight codes", qp.w_code[j] + so, 16, wc, n0, qm0, wave, lane, st))
                                    return false;
                            if (!in_range("quarter token codes", qp.x_code + so, 16, xc, n0, qm0, wave, lane, st))
                                return false;
                            if (!in_range("quarter weight scales", qp.w_scale + so, 4, ws, n0, qm0, wave, lane, st))
                                return false;
                            if (!in_range("quarter token scales", qp.x_scale + so, 4, xs, n0, qm0, wave, lane, st))
                                return false;
                        }
                    }
                }
        }
    return true;
}

int main(int argc, char** argv) {
    int i = 1;
    bool unclamped = false;
    if (i < argc && std::strcmp(argv[i], "--unclamped") == 0) {
        unclamped = true;
        ++i;
    }
    if ((argc - i) % 3 != 0 || argc - i == 0) {
        std::fprintf(stderr, "usage: %s [--unclamped] M N K [M N K ...]\n", argv[0]);
        return 2;
    }
    for (; i < argc; i += 3) {
        const int M = std::atoi(argv[i]), N = std::atoi(argv[i + 1]), K = std::atoi(argv[i + 2]);
        g_checked = 0;
        if (!check_shape(M, N, K, unclamped)) return 1;
        std::printf("ok %d %d %d: %lld loads\n", M, N, K, g_checked);
    }
    return 0;
}
