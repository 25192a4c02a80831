// gemm_epi_prep.hpp -- launchers of the operand preparation passes
// (gemm_epi_prep.hip) that uint8 inputs and widened fp8 inputs need.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

// For the uint8 operand x (L batches of R rows by K; x[l][r][k] when kmajor,
// else x[l][k][r] with R a multiple of 16): flipped gets x with every byte's
// top bit flipped (the same layout), sums[l][r] the sum over k of the
// unsigned bytes.  Enqueued on stream s; for an MN-major operand a fill
// kernel zeroes sums first.
void launch_u8_prep(const uint8_t* x, bool kmajor, int64_t L, int64_t R, int64_t K, uint8_t* flipped,
                    int32_t* sums, hipStream_t s);

// out[i] = the fp8 value x[i] (e4m3, or e5m2 when e5m2) as fp16, exactly, for
// i < n (n a multiple of 16).  Enqueued on stream s.
void launch_f8_widen(const uint8_t* x, int64_t n, bool e5m2, uint16_t* out, hipStream_t s);

}  // namespace gemm_epi
