/*
 * mla_verify_probe.h -- measurement helper built beside the verify library
 * (libmla_verify_probe.so); not part of the verify operation.
 *
 * The benchmark reports the verify kernels' throughput against the published
 * dense bf16 MFMA peak and against the MFMA throughput this GPU sustains under
 * a pure MFMA load, which this probe measures.
 */
#ifndef MLA_VERIFY_PROBE_H
#define MLA_VERIFY_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launches `grid` workgroups of 256 threads (four waves, one per SIMD), each
 * wave issuing iters x mlav_probe_mfma_per_wave() independent
 * v_mfma_f32_32x32x16_bf16 (32768 flop each) on `stream`, asynchronously.
 *   out     [grid * 256] fp32 DEVICE: a value per thread (keeps the work live)
 *   cycles  [grid * 4] uint64 DEVICE: shader-clock cycles of each wave's loop
 * grid 1 .. 2^20, iters 1 .. 2^24. Returns 0, 2 (bad argument) or 7 (HIP launch error).
 */
int32_t mlav_probe_mfma(int32_t grid, int32_t iters, float* out, unsigned long long* cycles, void* stream);

/* MFMA instructions per loop iteration per wave. */
int32_t mlav_probe_mfma_per_wave(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_PROBE_H */
