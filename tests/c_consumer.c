/*
 * A plain C consumer of libfp4dit.so (C99, no C++), the way a host program
 * that is not Python would drive the library: it creates its own HIP stream
 * and device buffers, then quantises activations, packs a weight and runs
 * the fused FP4 GEMM + per-head RMSNorm through the C ABI (include/fp4dit.h).
 * Built by python -m fp4_diffusion_transformer_amd.build next to this file;
 * tests/test_gpu_c_consumer.py runs it and checks its output against the
 * oracle.
 *
 *   c_consumer DIR M N K [swiglu]
 *
 * reads DIR/x.bin (bf16 bits, [M][K]) and DIR/w.bin (fp32, [K][N]).
 * Default: also DIR/g.bin (fp32 gains, [N]); writes DIR/y.bin (bf16 bits,
 * [M][N]) = per-head (128) RMSNorm of the MXFP4 GEMM, gains on every
 * column, eps 1e-6.  "swiglu": w is [gate | up] (N/2 columns each), packed
 * with the library's interleave group; writes the MXFP4 requantisation of
 * SwiGLU(x.W) as DIR/codes.bin and DIR/scales.bin (MX_TILED, [M][N/2]).
 * Exit status 0 on success; a failing call prints its status.
 */
#include <stdio.h>
#include <stdlib.h>

#include "fp4dit.h"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
            return 1;                                                          \
        }                                                                      \
    } while (0)
#define FP4_OK(x)                                                              \
    do {                                                                       \
        fp4dit_status s_ = (x);                                                \
        if (s_ != FP4DIT_OK) {                                                 \
            fprintf(stderr, "%s: %s\n", #x, fp4dit_status_string(s_));         \
            return 1;                                                          \
        }                                                                      \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

int main(int argc, char** argv) {
    if (argc != 5 && argc != 6) {
        fprintf(stderr, "usage: %s DIR M N K [swiglu]\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    const int64_t M = atoll(argv[2]), N = atoll(argv[3]), K = atoll(argv[4]);
    const int swiglu = argc == 6;
    uint16_t* x = read_file(dir, "x.bin", (size_t)(M * K) * 2);
    float* w = read_file(dir, "w.bin", (size_t)(K * N) * 4);
    float* g = swiglu ? malloc(4) : read_file(dir, "g.bin", (size_t)N * 4);
    if (!x || !w || !g) {
        fprintf(stderr, "cannot read the inputs in %s\n", dir);
        return 1;
    }
    /* MX_TILED buffers: codes padded to an even row count, scales to 32 rows */
    const size_t a_codes = round_up((size_t)M, 2) * (size_t)(K / 2), a_scales = round_up((size_t)M, 32) * (size_t)(K / 32);
    const size_t b_codes = round_up((size_t)N, 2) * (size_t)(K / 2), b_scales = round_up((size_t)N, 32) * (size_t)(K / 32);
    void *dx, *dw, *dg, *dy;
    uint8_t *dac, *das, *dbc, *dbs;
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    HIP_OK(hipMalloc(&dx, (size_t)(M * K) * 2));
    HIP_OK(hipMalloc(&dw, (size_t)(K * N) * 4));
    HIP_OK(hipMalloc(&dg, (size_t)N * 4));
    HIP_OK(hipMalloc(&dy, (size_t)(M * N) * 2));
    HIP_OK(hipMalloc((void**)&dac, a_codes));
    HIP_OK(hipMalloc((void**)&das, a_scales));
    HIP_OK(hipMalloc((void**)&dbc, b_codes));
    HIP_OK(hipMalloc((void**)&dbs, b_scales));
    HIP_OK(hipMemcpyAsync(dx, x, (size_t)(M * K) * 2, hipMemcpyHostToDevice, st));
    HIP_OK(hipMemcpyAsync(dw, w, (size_t)(K * N) * 4, hipMemcpyHostToDevice, st));
    HIP_OK(hipMemcpyAsync(dg, g, (size_t)N * 4, hipMemcpyHostToDevice, st));

    FP4_OK(fp4dit_quantize_mxfp4(dx, FP4DIT_BF16, M, K, dac, das, FP4DIT_MX_TILED, st));
    if (swiglu) {
        const int64_t nh = N / 2;
        const size_t h_codes = round_up((size_t)M, 2) * (size_t)(nh / 2), h_scales = round_up((size_t)M, 32) * (size_t)(nh / 32);
        uint8_t *dhc, *dhs;
        HIP_OK(hipMalloc((void**)&dhc, h_codes));
        HIP_OK(hipMalloc((void**)&dhs, h_scales));
        FP4_OK(fp4dit_pack_weight(dw, FP4DIT_F32, K, N, fp4dit_swiglu_interleave_group(), dbc, dbs,
                                  FP4DIT_MX_TILED, st));
        FP4_OK(fp4dit_gemm_fp4_epilogue_swiglu(M, N, K, dac, das, dbc, dbs, NULL, FP4DIT_BF16, dhc, dhs, st));
        uint8_t* hc = malloc(h_codes);
        uint8_t* hs = malloc(h_scales);
        if (!hc || !hs) return 1;
        HIP_OK(hipMemcpyAsync(hc, dhc, h_codes, hipMemcpyDeviceToHost, st));
        HIP_OK(hipMemcpyAsync(hs, dhs, h_scales, hipMemcpyDeviceToHost, st));
        HIP_OK(hipStreamSynchronize(st));
        char path[4096];
        snprintf(path, sizeof path, "%s/codes.bin", dir);
        FILE* f = fopen(path, "wb");
        if (!f || fwrite(hc, 1, h_codes, f) != h_codes) return 1;
        fclose(f);
        snprintf(path, sizeof path, "%s/scales.bin", dir);
        f = fopen(path, "wb");
        if (!f || fwrite(hs, 1, h_scales, f) != h_scales) return 1;
        fclose(f);
        hipFree(dhc); hipFree(dhs);
        free(hc); free(hs);
        return 0;
    }
    FP4_OK(fp4dit_pack_weight(dw, FP4DIT_F32, K, N, 0, dbc, dbs, FP4DIT_MX_TILED, st));
    FP4_OK(fp4dit_gemm_fp4_epilogue_rmsnorm_head(M, N, K, dac, das, dbc, dbs, 128, N, (const float*)dg, 1e-6f,
                                                 dy, FP4DIT_BF16, st));

    uint16_t* y = malloc((size_t)(M * N) * 2);
    if (!y) return 1;
    HIP_OK(hipMemcpyAsync(y, dy, (size_t)(M * N) * 2, hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    char path[4096];
    snprintf(path, sizeof path, "%s/y.bin", dir);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(y, 2, (size_t)(M * N), f) != (size_t)(M * N)) {
        fprintf(stderr, "cannot write %s\n", path);
        return 1;
    }
    fclose(f);
    hipFree(dx); hipFree(dw); hipFree(dg); hipFree(dy);
    hipFree(dac); hipFree(das); hipFree(dbc); hipFree(dbs);
    hipStreamDestroy(st);
    free(x); free(w); free(g); free(y);
    return 0;
}
