/*
 * fmha_microbench.h -- instruction-throughput microbenchmarks for gfx950.
 *
 * Measurement support, not part of the attention boundary (fmha.h): it backs
 * the FMHA kernels' design with the rates the hardware actually sustains.
 * "Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV, GB300)", section 1:
 * measure each instruction's throughput in isolation, with independent
 * dependency chains and a cycle counter around the timed loop, before
 * budgeting a kernel with it. The rates that matter for the attention forward
 * pass are those of its softmax (exp2, FMA, the P conversions to bf16, e4m3
 * and e2m1, exp2 mixed with e4m3 conversion), of its products (bf16 and fp8
 * MFMA), and of the LDS operand reads that feed them.
 *
 * Library: libfmha_microbench.so (built next to libfmha.so).
 */
#ifndef FMHA_MICROBENCH_H_
#define FMHA_MICROBENCH_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Benchmarks. Each wave of one workgroup per compute unit (4 * waves_per_simd
 * waves, i.e. waves_per_simd on each SIMD) runs a timed loop; "cycles" are
 * shader-clock cycles (s_memtime) of one wave. */
#define FMHA_MB_EXP2 0          /* v_exp_f32, 8 chains                           */
#define FMHA_MB_FMA 1           /* v_fma_f32, 8 chains                           */
#define FMHA_MB_CVT_BF16 2      /* v_cvt_pk_bf16_f32 (2 floats -> packed bf16)   */
#define FMHA_MB_CVT_E4M3 3      /* v_cvt_pk_fp8_f32 (2 floats -> 2 e4m3)         */
#define FMHA_MB_CVT_E2M1 4      /* v_cvt_scalef32_pk_fp4_f32 (2 floats -> 2 e2m1) */
#define FMHA_MB_EXP2_E4M3 5     /* one op = 2 v_exp_f32 + 1 v_cvt_pk_fp8_f32     */
#define FMHA_MB_MFMA_BF16 6     /* v_mfma_f32_32x32x16_bf16, 4 accumulators      */
#define FMHA_MB_MFMA_E4M3 7     /* v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3) */
#define FMHA_MB_LDS_B128 8      /* ds_read_b128, conflict-free, 1 KB per wave op  */
#define FMHA_MB_MFMA_LDS_B128 9 /* bf16 MFMA whose A operand (1 KB) each MFMA
                                   reads from LDS, 16 reads ahead               */
#define FMHA_MB_MFMA_WITH_VALU 10 /* per SIMD, wave 0 runs bf16 MFMAs while wave
                                     1 runs a softmax-like vector stream (32
                                     scores: FMA, exp2, sum, bf16 pack);
                                     waves_per_simd must be 2                   */
#define FMHA_MB_SOFTMAX 11      /* that softmax-like vector stream alone; one
                                   op = one iteration (32 scores)               */
#define FMHA_MB_EXP2_POLY 12     /* 2^x on the FMA path: range reduction and a
                                   degree-3 polynomial, 8 vector instructions;
                                   one op = one 2^x                             */
#define FMHA_MB_EXP2_WITH_FMA 13 /* one op = 1 v_exp_f32 + 4 v_fma_f32 on
                                   independent chains                           */
#define FMHA_MB_COUNT 14

/*
 * Run benchmark `which` on the current HIP device: one warm-up launch, then
 * one measured launch of `iters` loop iterations, synchronously (this call
 * allocates a small device buffer, launches on the null stream and waits).
 *
 *   which           FMHA_MB_*
 *   waves_per_simd  1 .. 4 (FMHA_MB_MFMA_WITH_VALU: exactly 2)
 *   iters           1 .. 2^20 loop iterations
 *   result          host array of 2 doubles, written on success:
 *                   [0] median over the device's waves of cycles per
 *                       instruction (per op for FMHA_MB_EXP2_E4M3,
 *                       FMHA_MB_SOFTMAX, FMHA_MB_EXP2_POLY and
 *                       FMHA_MB_EXP2_WITH_FMA; for FMHA_MB_MFMA_WITH_VALU, of
 *                       the MFMA waves)
 *                   [1] FMHA_MB_MFMA_WITH_VALU: median cycles per iteration
 *                       of the vector waves' stream; otherwise 0
 *
 * Returns 0 on success, 1 for an invalid argument (nothing is launched),
 * 3 when a HIP call fails.
 */
int32_t fmha_microbench_run(int32_t which, int32_t waves_per_simd, int32_t iters,
                            double* result);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_MICROBENCH_H_ */
