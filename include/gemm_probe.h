/*
 * libgemm_probe: measurement probes beside libgemm (not GEMMs).
 *
 * The matrix-core rate a GEMM can reach is capped by the clock that the
 * chip's power limit allows under that load, which falls below the
 * nominal 2.4 GHz with the 16-bit instructions.  These probes measure the
 * cap on the device that runs them, so that a GEMM's rate can be set
 * against what the same instruction sustains with no memory traffic.
 *
 * Both probes launch 256 workgroups (gemm_probe_workgroups(), one per CU)
 * on `stream` (a hipStream_t; NULL = default stream), asynchronously.
 * `stamps` is a device buffer of 4 x 256 uint64: for workgroup w,
 * stamps[4w + 0] and [4w + 2] are the shader-cycle counter (s_memtime) at
 * start and end, stamps[4w + 1] and [4w + 3] the 100 MHz constant clock
 * (s_memrealtime) at start and end; the workgroup's clock is
 * (stamps[4w+2] - stamps[4w]) / (stamps[4w+3] - stamps[4w+1]) x 100 MHz.
 * `sink` is a device buffer of floats that keeps the work observable
 * (256 x 256 for the MFMA probe, 256 x 64 for the clock probe); its
 * contents are meaningless.  Return: 0 on success, -1 for bad arguments
 * (negative count, NULL buffer, unknown dtype), -3 for a launch error.
 */
#ifndef GEMM_PROBE_H
#define GEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t gemm_probe_workgroups(void);

/* Matrix-core stream with operands in registers: `steps` k steps of 16
 * instructions per wave (4 waves per workgroup, one 128 x 128 block of
 * 32 x 32 accumulators each), dtype 0 FP32 (v_mfma_f32_32x32x2_f32),
 * 1 FP16 and 2 BF16 (v_mfma_f32_32x32x16_*), 3 FP8 E4M3 and 4 FP8 E5M2
 * (v_mfma_f32_32x32x64_f8f6f4); `steps` even.  Flops: 256 x 4 x steps x
 * 16 x 2 x 32 x 32 x k, with k = 2, 16, 16, 64, 64. */
int32_t gemm_probe_mfma(int32_t dtype, int64_t steps, uint64_t *stamps, float *sink, void *stream);

/* The same stream with the 16 x 16 instructions (v_mfma_f32_16x16x4_f32,
 * v_mfma_f32_16x16x32_f16 / _bf16, v_mfma_f32_16x16x128_f8f6f4): 8 x 8
 * blocks of 4 accumulators per wave, one k step of 64 instructions per two
 * `steps`, so the flops are those of gemm_probe_mfma with the same `steps`;
 * `steps` even. */
int32_t gemm_probe_mfma16(int32_t dtype, int64_t steps, uint64_t *stamps, float *sink, void *stream);

/* A dependent FMA loop of `iters` trips per lane (64 lanes per workgroup):
 * the shader clock with little power drawn, or right after another kernel
 * on the same stream. */
int32_t gemm_probe_clock(int64_t iters, uint64_t *stamps, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_PROBE_H */
