/*
 * mla_verify_probe.h -- measurement helper built beside the verify library
 * (libmla_verify_probe.so); not part of the verify operation.
 *
 * The benchmark reports the verify kernels' throughput against the published
 * dense bf16 MFMA peak and against the MFMA throughput this GPU sustains under
 * a pure MFMA load, which the first probe measures; the second measures what
 * the split kernel's loop step costs as a bare data flow.
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

/* Parts of mlav_probe_step_mix beyond its 50 MFMAs per wave and step. */
#define MLAV_MIX_LDS 1      /* MFMA A operands read from LDS: 18 128-bit reads (score product) and
                               32 transposing 64-bit reads (value product) per wave and step */
#define MLAV_MIX_DMA 2      /* nine 1 KB direct-to-LDS buffer loads per wave and step, three steps ahead */
#define MLAV_MIX_BARRIERS 4 /* two workgroup barriers per step */
#define MLAV_MIX_SRC_BYTES (64u << 20) /* bytes of `src` the loads read */

/*
 * The split kernel's loop step (one 32-key tile) as a bare data flow: the same
 * MFMAs, LDS operand reads, tile loads and barriers per wave, with no softmax
 * and no data dependency between the products. Launches `grid` workgroups of
 * 256 threads (four waves, one per SIMD) on `stream`, asynchronously, each
 * running iters x mlav_probe_steps_per_iteration() steps.
 *   parts   bit mask of MLAV_MIX_* (0..7)
 *   src     DEVICE buffer of at least MLAV_MIX_SRC_BYTES, read by the loads
 *   out     [grid * 256] fp32 DEVICE: a value per thread (keeps the work live)
 *   cycles  [grid * 4] uint64 DEVICE: shader-clock cycles of each wave's loop
 * grid 1 .. 2^20, iters 1 .. 2^20. Returns 0, 2 (bad argument) or 7 (HIP launch error).
 */
int32_t mlav_probe_step_mix(int32_t grid, int32_t iters, int32_t parts, const void* src, float* out,
                            unsigned long long* cycles, void* stream);

/* Loop steps per iteration of mlav_probe_step_mix. */
int32_t mlav_probe_steps_per_iteration(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_PROBE_H */
