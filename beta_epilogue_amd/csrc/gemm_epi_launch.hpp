// gemm_epi_launch.hpp -- host-side launcher of one kernel variant.  Defined
// and explicitly instantiated per variant in gemm_epi_part.hip; the variant
// table in gemm_epi.hip refers to the instantiations.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_epi_kernel.hpp"

namespace gemm_epi {

// Launches gemm_epi_kernel<CF> on `grid` workgroups of CF::THREADS threads
// on stream s (errors are read back with hipGetLastError by the caller).
template <class CF>
void launch(const Params& p, int grid, hipStream_t s);

}  // namespace gemm_epi
