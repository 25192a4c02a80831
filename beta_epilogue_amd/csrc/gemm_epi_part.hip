// gemm_epi_part.hip -- compiles the kernel variants of gemm_epi_variants.inc
// whose `part` equals GEMM_EPI_PART (the build compiles this file once per
// part, in parallel, and links the objects with gemm_epi.hip).
#include "gemm_epi_launch.hpp"

#ifndef GEMM_EPI_PART
#error "GEMM_EPI_PART must be defined (0 .. 15)"
#endif

namespace gemm_epi {

template <class CF>
void launch(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_epi_kernel<CF>, dim3(grid), dim3(CF::THREADS), 0, s, p);
}

#define GEMM_EPI_INSTANTIATE(...) template void launch<Cfg<__VA_ARGS__>>(const Params&, int, hipStream_t);
#define GEMM_EPI_SKIP(...)
#define GEMM_EPI_PICK_0 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_1 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_2 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_3 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_4 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_5 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_6 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_7 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_8 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_9 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_10 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_11 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_12 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_13 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_14 GEMM_EPI_SKIP
#define GEMM_EPI_PICK_15 GEMM_EPI_SKIP
#if GEMM_EPI_PART == 0
#undef GEMM_EPI_PICK_0
#define GEMM_EPI_PICK_0 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 1
#undef GEMM_EPI_PICK_1
#define GEMM_EPI_PICK_1 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 2
#undef GEMM_EPI_PICK_2
#define GEMM_EPI_PICK_2 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 3
#undef GEMM_EPI_PICK_3
#define GEMM_EPI_PICK_3 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 4
#undef GEMM_EPI_PICK_4
#define GEMM_EPI_PICK_4 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 5
#undef GEMM_EPI_PICK_5
#define GEMM_EPI_PICK_5 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 6
#undef GEMM_EPI_PICK_6
#define GEMM_EPI_PICK_6 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 7
#undef GEMM_EPI_PICK_7
#define GEMM_EPI_PICK_7 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 8
#undef GEMM_EPI_PICK_8
#define GEMM_EPI_PICK_8 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 9
#undef GEMM_EPI_PICK_9
#define GEMM_EPI_PICK_9 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 10
#undef GEMM_EPI_PICK_10
#define GEMM_EPI_PICK_10 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 11
#undef GEMM_EPI_PICK_11
#define GEMM_EPI_PICK_11 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 12
#undef GEMM_EPI_PICK_12
#define GEMM_EPI_PICK_12 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 13
#undef GEMM_EPI_PICK_13
#define GEMM_EPI_PICK_13 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 14
#undef GEMM_EPI_PICK_14
#define GEMM_EPI_PICK_14 GEMM_EPI_INSTANTIATE
#elif GEMM_EPI_PART == 15
#undef GEMM_EPI_PICK_15
#define GEMM_EPI_PICK_15 GEMM_EPI_INSTANTIATE
#else
#error "GEMM_EPI_PART out of range"
#endif
#define GEMM_EPI_CAT(a, b) a##b
#define X(PART, AB, AK, BK, CDN, BM, BN, RB, WM, WN, S, DS, BL, NAME) \
  GEMM_EPI_CAT(GEMM_EPI_PICK_, PART)(AB, AK, BK, CDN, BM, BN, RB, WM, WN, S, DS, BL)
#include <gemm_epi_variants.inc>  // (angle brackets: a partial build can put its own table first)
#undef X

}  // namespace gemm_epi
