// gemm_epi_u8.hpp -- launcher of the uint8 operand preparation (gemm_epi_u8.hip).
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

}  // namespace gemm_epi
