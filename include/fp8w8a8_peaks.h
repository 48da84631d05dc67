/* Measured peaks for the benchmark (libfp8w8a8_peaks.so): the FP8 MFMA rate
 * and the HBM read rate that this GPU sustains, reported beside the
 * published peaks (MI355X: 5.0 PFLOP/s dense FP8, 8 TB/s HBM3E).  Benchmark
 * tooling, not part of the Linear: the kernels compute nothing the method
 * defines.
 *
 * All pointers are device pointers; `stream` is a hipStream_t passed as
 * void*.  Calls only launch (no allocation, no synchronization); they return
 * 0 on success, 1 for a null pointer, 2 for a size out of range, 3 for a
 * misaligned pointer, 7 if the launch failed. */
#ifndef FP8W8A8_PEAKS_H
#define FP8W8A8_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Floats `out` must hold for fp8w8a8_peaks_mfma_loop over `workgroups`. */
int64_t fp8w8a8_peaks_mfma_out_floats(int64_t workgroups);

/* A loop of v_mfma_f32_32x32x64_f8f6f4 on register operands: `workgroups`
 * workgroups of 4 waves, each wave 8 independent accumulators x `iters`
 * MFMAs.  out: fp8w8a8_peaks_mfma_out_floats(workgroups) floats (the summed
 * accumulators, so that the work is live).  clk: 2 counters written by the
 * first wave: shader-clock cycles and 100 MHz reference ticks between its
 * start and end (their ratio x 100 MHz is the clock it ran at).
 * workgroups in [1, 2^20], iters >= 1. */
int fp8w8a8_peaks_mfma_loop(float* out, unsigned long long* clk, int64_t workgroups,
                            int iters, void* stream);

/* Flops of one fp8w8a8_peaks_mfma_loop launch (2 * 32 * 32 * 64 per MFMA). */
int64_t fp8w8a8_peaks_mfma_flops(int64_t workgroups, int iters);

/* Workgroups (and so uint32 outputs / 256) of a read of `bytes`: a fixed
 * 1024 (4 per compute unit), each stepping over the buffer. */
int64_t fp8w8a8_peaks_read_workgroups(int64_t bytes);

/* Streams `bytes` (a multiple of 16, src 16-byte aligned) from src, once,
 * with 16-byte nontemporal loads; out: fp8w8a8_peaks_read_workgroups(bytes) * 256
 * uint32 (the XOR of what each thread read). */
int fp8w8a8_peaks_read_stream(const void* src, int64_t bytes, uint32_t* out,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_PEAKS_H */
