/* drla_peaks.h -- attainable-peak measurement kernels (libdrla_peaks.so).
 *
 * Two microbenchmarks that price the prefill kernels' roofline against what
 * this chip actually sustains, beside its published peaks: a streaming copy
 * (HBM bandwidth) and independent chains of dependent MFMAs (matrix-core
 * throughput).  They compute nothing of the method and are not called by
 * the prefill path; the benchmark times them with HIP events on `stream`.
 *
 * All pointers are device pointers; `stream` is a hipStream_t passed as
 * void* (NULL: the null stream).  Launches are asynchronous; the return
 * value is 0 (launched), 1 (invalid argument, nothing launched) or 2 (a HIP
 * call failed).
 */
#ifndef DRLA_PEAKS_H
#define DRLA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes): one 16-byte non-temporal load and
 * store per thread, one 256-thread workgroup per 4 KiB.  `bytes` must be a
 * positive multiple of 16, at most 2^31 workgroups' worth, and src, dst
 * 16-byte aligned and disjoint.  The caller owns both buffers. */
int drla_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Matrix-core throughput: `blocks` workgroups of 256 threads (blocks <= 0:
 * 8 per compute unit), every wave runs `iters` rounds of 8 independent
 * accumulator chains, each round one MFMA per chain (kind 0: bf16
 * v_mfma_f32_16x16x32_bf16, 16384 flops each; 1: fp16 16x16x32, 16384;
 * 2: fp32 v_mfma_f32_16x16x4_f32, 2048).  Each wave writes its 64 lanes'
 * sums to out (out holds blocks * 256 floats, owned by the caller), so no
 * product is dead code.  *flops (if not NULL) receives the launch's
 * floating-point operation count; *grid (if not NULL) the block count used.
 * iters must be positive. */
int drla_peak_mfma(float* out, int kind, int iters, int blocks, void* stream, double* flops,
                   int* grid);

/* Workgroups drla_peak_mfma launches for `blocks` (resolving blocks <= 0);
 * 0 on error.  Lets the caller size `out`. */
int drla_peak_mfma_grid(int blocks);

#ifdef __cplusplus
}
#endif

#endif /* DRLA_PEAKS_H */
