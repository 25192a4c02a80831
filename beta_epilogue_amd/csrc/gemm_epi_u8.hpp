// gemm_epi_u8.hpp -- launcher of the uint8 row/column sums (gemm_epi_u8.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

// out[l][r] = sum over k of the uint8 operand x (L batches of R rows by K):
// x[l][r][k] when kmajor, else x[l][k][r] (R a multiple of 16).  Enqueued on
// stream s; for an MN-major operand a fill kernel zeroes out first.
void launch_u8_sums(const uint8_t* x, bool kmajor, int64_t L, int64_t R, int64_t K, int32_t* out,
                    hipStream_t s);

}  // namespace gemm_epi
