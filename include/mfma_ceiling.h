/* mfma_ceiling.h -- measurement tool shipped beside the GEMM library
 * (libmfma_ceiling.so); not part of the GEMM path.
 *
 * Measures the steady shader clock and throughput of a register-only stream
 * of v_mfma_f32_32x32x16_f16 or v_mfma_f32_16x16x32_f16 (8 waves per CU,
 * 8 or 16 independent accumulators per wave, one workgroup per CU of the
 * current HIP device), with constant or with uniformly random fp16 operands.  Under the board power cap the
 * clock depends on the operand data, so this is the attainable MFMA rate for
 * data of a given kind; bench.py --mfma-ceiling reports both.
 */
#ifndef MFMA_CEILING_H
#define MFMA_CEILING_H

#ifdef __cplusplus
extern "C" {
#endif

/* block: 32 (32x32x16) or 16 (16x16x32); anything else returns
 *   hipErrorInvalidValue.
 * random_operands: 0 = every fp16 operand is 1.0; 1 = uniform in sign,
 *   exponent 2^-1 .. 2^-4 and mantissa (seeded xorshift64, fixed seed).
 * iters: MFMAs per accumulator per launch (rounded down to a multiple of 8).
 * reps: timed launches after one short warm-up launch; the last is reported.
 * Outputs (host pointers, caller-owned): *ms = HIP-event time of the last
 *   launch, *ghz = shader clock of workgroup 0 (clock64 against the 100 MHz
 *   wall clock), *tflops = 2*32*32*16 FLOP per MFMA over *ms.
 * Allocates and frees its own device buffers (~16 MB).  Returns 0, or the
 * hipError_t of the first failing HIP call (outputs then unset). */
int mfma_ceiling_run(int block, int random_operands, int iters, int reps, float* ms, double* ghz,
                     double* tflops);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_CEILING_H */
