// gemm_epi_splitk.hpp -- the split-K reduction + epilogue kernel's arguments
// and launcher (gemm_epi_splitk.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

// Element type codes: the public header's numbers.
enum : int { SK_F16 = 1, SK_BF16 = 2, SK_F32 = 5, SK_I32 = 6 };

struct SplitkParams {
  const void* ws;   // splits * tail_tiles slots of tile_m*tile_n fp32 (int32)
                    // partial sums: slot s*tail_tiles + j is slice s of tile
                    // dp_tiles + j (raster order), its rows x cols inside the
                    // matrix packed in D's majorness
  const void* C;    // NULL when the beta term is skipped
  const void* X;    // NULL when the x_factor term is skipped
  void* D;
  void* Y;          // NULL when Y is not written
  int64_t M, N;
  int32_t dp_tiles, tail_tiles;
  int32_t tiles_m, tiles_n, group_m;  // the GEMM's raster
  int32_t tile_m, tile_n;             // multiples of 4
  int32_t cd_nmajor;                  // C/X/D/Y (and the slots) N-major
  int32_t splits;
  int32_t c_dtype, x_dtype, d_dtype, y_dtype;
  int32_t int_path;  // int8 inputs: int32 sums and epilogue
  float alpha, beta, xf;
  int32_t ialpha, ibeta, ix;
  int32_t relu;
};

// Enqueues the kernel on `grid` workgroups of 256 threads on stream s.
void launch_splitk_epilogue(const SplitkParams& p, int grid, hipStream_t s);

}  // namespace gemm_epi
