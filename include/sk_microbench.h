/* sk_microbench.h -- the machine's own peaks, for reporting measured rates
 * against what this MI355X sustains rather than only against its spec sheet.
 *
 * Not part of the GEMM path: libskmb.so is a separate library that bench.py
 * loads to time these kernels with HIP events on the stream it launches them
 * on.  Both entry points launch asynchronously on `stream` and return a
 * hipError_t value (0 = hipSuccess).
 */
#ifndef SK_MICROBENCH_H
#define SK_MICROBENCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA issue rate: `grid` workgroups of 256 threads (4 waves); every wave
 * runs `rounds` rounds of 8 independent MFMAs of one type (four A times two
 * B operand fragments of hashed values, fixed across rounds; accumulators in
 * registers):
 *   dtype 0: v_mfma_f32_16x16x4_f32   (2 * 16 * 16 * 4  = 2048 flop each)
 *   dtype 1: v_mfma_f32_32x32x16_f16  (2 * 32 * 32 * 16 = 32768 flop each)
 *   dtype 2: v_mfma_f32_32x32x16_bf16 (32768 flop each)
 * so one launch does grid * 4 * rounds * 8 MFMAs.  `sink` (device, grid * 256
 * floats, caller-owned) receives each thread's accumulator sum so the work
 * cannot be removed.  Two workgroups per CU (grid = 2 x CUs) put two waves on
 * every SIMD, as the GEMM kernels run.  Returns hipErrorInvalidValue for an
 * unknown dtype, non-positive sizes or `rounds` not a multiple of 4 (the
 * loop runs four rounds per pass). */
int skmb_mfma(int dtype, int rounds, int grid, float *sink, hipStream_t stream);

/* HBM read rate: `grid` workgroups of 256 threads read `bytes` bytes at
 * `src` (device, 16-byte aligned, bytes a multiple of 16) once: each wave
 * takes 8 KiB blocks in turn (eight 1 KiB loads in flight, 16 bytes per
 * lane), and XORs what it read into `sink` (device, grid * 256 uint32,
 * caller-owned).
 * Returns hipErrorInvalidValue for misaligned or non-positive sizes. */
int skmb_read(const void *src, int64_t bytes, int grid, uint32_t *sink, hipStream_t stream);

/* LDS read rate: `grid` workgroups of 256 threads (4 waves), each filling
 * 32 KiB of LDS and then running `rounds` rounds of 8 reads per wave:
 *   mode 0: 16 bytes per lane (1 KiB per read instruction, conflict-free),
 *   mode 1: 8 bytes per lane by the transposing read ds_read_b64_tr_b16
 *           (512 bytes per instruction),
 * so one launch reads grid * 4 * rounds * 8 * (1024 or 512) bytes of LDS.
 * Two workgroups per CU (grid = 2 x CUs) put eight waves on every CU, as the
 * 256 x 256 GEMM kernel runs.  `sink` (device, grid * 256 uint32,
 * caller-owned) receives each thread's XOR of what it read.  Returns
 * hipErrorInvalidValue for an unknown mode or non-positive sizes. */
int skmb_lds(int mode, int rounds, int grid, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
