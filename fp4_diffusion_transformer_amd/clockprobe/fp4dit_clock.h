/*
 * fp4dit_clock.h - C ABI of libfp4dit_clock.so, a measurement helper kept out
 * of the method's library (libfp4dit.so): the shader clock under a scaled FP4
 * MFMA load, used to quote the MXFP4 roofline at the clock a box sustains.
 */
#ifndef FP4DIT_CLOCK_H
#define FP4DIT_CLOCK_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * `workgroups` workgroups of 4 waves (one per CU loads the whole chip, as
 * the persistent GEMM does) each run `iters` rounds of 16 independent
 * 32x32x64 FP4 MFMAs on pseudo-random operands.  Wave w writes, to the
 * caller-owned device buffer `out` (3 uint64 per wave, 8-byte aligned):
 * out[3w] the ticks of the shader-clock counter (s_memtime) and out[3w + 1]
 * those of the constant 100 MHz counter (s_memrealtime) over its MFMAs,
 * out[3w + 2] a checksum.  Its clock in GHz is 0.1 * out[3w] / out[3w + 1].
 * Enqueued on `stream`; the caller synchronises.  Returns 0 on success, 1
 * for a NULL `out`, 3 for a misaligned one, 2 unless 1 <= workgroups <= 65536
 * and 1 <= iters <= 2^20, 5 if the launch failed (the status values of
 * include/fp4dit.h).
 */
int32_t fp4dit_clock_probe(uint64_t* out, int32_t workgroups, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4DIT_CLOCK_H */
