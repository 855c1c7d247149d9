/*
 * fp4probe.h - C ABI of the measurement probe that ships beside libfp4lin.so (libfp4probe.so).
 *
 * The FP4 GEMM of the linear forward (QbitAI report on "Optimizing Large Language Model
 * Training Using FP4 Quantization", GEMM-kernel paragraph) is priced against the chip's dense
 * FP4 matrix peak.  This probe measures what the matrix cores of the present device actually
 * sustain when they do nothing else: every wave issues a long chain of independent
 * V_MFMA_SCALE_F32_32X32X64_F8F6F4 instructions on FP4 operands held in registers (no memory
 * traffic inside the timed loop; the unscaled form with unit block scales, as the GEMM
 * issues it), and reads the shader clock counter and the constant-rate
 * real-time counter before and after, so the caller can derive the clock the loop ran at.
 *
 * Not part of the forward: only the benchmark calls it.
 */
#ifndef FP4PROBE_H
#define FP4PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` workgroups of 256 threads (4 waves) on `stream` (hipStream_t as void*).
 * Each wave runs `iters` iterations of 8 independent 32x32x64 FP4 MFMAs (131072 FLOP each),
 * i.e. blocks * 4 * iters * 8 * 131072 FLOP in all.
 *   clocks  device uint64[blocks * 4 * 4] (out): per wave, the shader-clock counter and the
 *           real-time counter (100 MHz) at the start and at the end of its loop, in the
 *           order start_clock, end_clock, start_real, end_real.
 *   sink    device float[blocks * 256] (out): a value derived from the accumulators, so the
 *           loop is not optimized away.
 * Returns 0, 1 for invalid arguments (blocks < 1, iters < 1, NULL pointers), or 2 if the
 * launch failed. */
int32_t fp4_probe_mfma_fp4(int32_t blocks, int32_t iters, uint64_t *clocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4PROBE_H */
