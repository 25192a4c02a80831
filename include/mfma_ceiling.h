/* mfma_ceiling.h -- measurement tool shipped beside the GEMM library
 * (libmfma_ceiling.so); not part of the GEMM path.
 *
 * Measures the steady shader clock and throughput of a register-only stream
 * of one MFMA instruction (8 waves per CU, 8 or 16 independent accumulators
 * per wave, one workgroup per CU of the current HIP device), with constant or
 * with random operands: v_mfma_f32_32x32x16_f16 / 16x16x32_f16, the bf16
 * pair, v_mfma_i32_32x32x32_i8 / 16x16x64_i8 and
 * v_mfma_scale_f32_32x32x64_f8f6f4 / 16x16x128_f8f6f4 on e4m3.  Under the
 * board power cap the clock depends on the operand data, so this is the
 * attainable MFMA rate for data of a given kind; bench.py --mfma-ceiling
 * reports both.
 */
#ifndef MFMA_CEILING_H
#define MFMA_CEILING_H

#ifdef __cplusplus
extern "C" {
#endif

/* type: the operand type, with gemm_epi.h's codes: 1 fp16, 2 bf16, 3 e4m3,
 *   4 int8; anything else returns hipErrorInvalidValue.
 * block: 32 (the 32x32 instruction) or 16 (two 16x16 instructions per 32x32
 *   one, the same FLOP); anything else returns hipErrorInvalidValue.
 * random_operands: 0 = every operand element is 1; 1 = seeded xorshift64
 *   data, fixed seed: fp16/bf16 uniform in sign, exponent 2^-1 .. 2^-4 and
 *   mantissa; int8 uniform over all 256 values; e4m3 uniform in sign,
 *   exponent field 0..8 and mantissa (|v| < 4).
 * iters: 32x32 steps per accumulator per launch (rounded down to a multiple
 *   of 8).
 * reps: timed launches after one short warm-up launch; the last is reported.
 * Outputs (host pointers, caller-owned): *ms = HIP-event time of the last
 *   launch, *ghz = shader clock of workgroup 0 (clock64 against the 100 MHz
 *   wall clock), *tflops = FLOP (OP for int8) of the 32x32 steps over *ms, in
 *   units of 10^12 per second.
 * Allocates and frees its own device buffers (~16 MB).  Returns 0, or the
 *   hipError_t of the first failing HIP call (outputs then unset). */
int mfma_ceiling_run_type(int type, int block, int random_operands, int iters, int reps, float* ms, double* ghz,
                          double* tflops);

/* mfma_ceiling_run_type with type 1 (fp16). */
int mfma_ceiling_run(int block, int random_operands, int iters, int reps, float* ms, double* ghz,
                     double* tflops);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_CEILING_H */
