// gemm_epi_u8.hip -- the sums along K that uint8 inputs need.
//
// uint8 A/B (the pipeline API card's "int8 / uint8 with int32") run on the
// int8 MFMA: every byte u is fed as the signed byte u - 128 (its top bit
// flipped), and since
//   sum_k u_a u_b = sum_k (u_a - 128)(u_b - 128) + 128 (sum_k u_a + sum_k u_b) - 16384 K,
// the int32 epilogue adds 128 times the sum along K of the output's A row and
// B column, and -16384 K (-16384 times K rounded up to whole K tiles: the
// MFMA also sums the zero bytes staged past K, flipped to -128 x -128; int32
// arithmetic wraps, so the result is exact whenever it fits).  These kernels compute those sums: rsum[l][r] = sum_k
// X[l][r][k] for a K-major operand (r = m or n), or sum_k X[l][k][r] for an
// M-major A / N-major B.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_epi_u8.hpp"

namespace gemm_epi {

namespace {

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// Sum of the four bytes of each word, added to acc.
__device__ __forceinline__ unsigned bytesum(v4u_t w, unsigned acc) {
  acc = __builtin_amdgcn_udot4(w.x, 0x01010101u, acc, false);
  acc = __builtin_amdgcn_udot4(w.y, 0x01010101u, acc, false);
  acc = __builtin_amdgcn_udot4(w.z, 0x01010101u, acc, false);
  return __builtin_amdgcn_udot4(w.w, 0x01010101u, acc, false);
}

// K-major: one wave per row, 16 bytes per lane and step (K bytes per row are
// a multiple of 16), then a sum across the wave.
__global__ __launch_bounds__(256) void sums_kmajor(const uint8_t* x, int64_t rows, int64_t K, int32_t* out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // over L * R rows
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const v4u_t* p = (const v4u_t*)(x + row * K);
  unsigned acc = 0;
  for (int64_t c = lane; c < K / 16; c += 64) acc = bytesum(__builtin_nontemporal_load(p + c), acc);
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) out[row] = (int32_t)acc;
}

// M-major A / N-major B: a thread owns 16 consecutive r (R is a multiple of
// 16) and a chunk of k-rows; its sums are added into out with atomics
// (out starts at zero).
__global__ __launch_bounds__(256) void sums_mnmajor(const uint8_t* x, int64_t R, int64_t K, int64_t kchunk,
                                                    int32_t* out) {
  const int64_t r16 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 16 r
  const int l = blockIdx.z;
  if (r16 * 16 >= R) return;
  const int64_t k0 = (int64_t)blockIdx.y * kchunk;
  const int64_t k1 = k0 + kchunk < K ? k0 + kchunk : K;
  const uint8_t* base = x + (int64_t)l * K * R + r16 * 16;
  unsigned s[16] = {};
  for (int64_t k = k0; k < k1; ++k) {
    const v4u_t w = __builtin_nontemporal_load((const v4u_t*)(base + k * R));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned v = w[j];
      s[4 * j + 0] += v & 0xff;
      s[4 * j + 1] += (v >> 8) & 0xff;
      s[4 * j + 2] += (v >> 16) & 0xff;
      s[4 * j + 3] += v >> 24;
    }
  }
  int32_t* o = out + (int64_t)l * R + r16 * 16;
#pragma unroll
  for (int j = 0; j < 16; ++j) atomicAdd(o + j, (int32_t)s[j]);
}

__global__ __launch_bounds__(256) void fill_zero(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace

void launch_u8_sums(const uint8_t* x, bool kmajor, int64_t L, int64_t R, int64_t K, int32_t* out,
                    hipStream_t s) {
  if (kmajor) {
    const int64_t rows = L * R;
    hipLaunchKernelGGL(sums_kmajor, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, rows, K, out);
  } else {
    const int64_t n = L * R;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                       s, out, n);
    const int64_t kchunk = 64;
    const dim3 grid((unsigned)((R / 16 + 255) / 256), (unsigned)((K + kchunk - 1) / kchunk), (unsigned)L);
    hipLaunchKernelGGL(sums_mnmajor, grid, dim3(256), 0, s, x, R, K, kchunk, out);
  }
}

}  // namespace gemm_epi
