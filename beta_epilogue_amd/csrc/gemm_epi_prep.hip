// gemm_epi_prep.hip -- the operand preparation passes that uint8 inputs and
// widened fp8 inputs need.
//
// uint8 A/B (the pipeline API card's "int8 / uint8 with int32") run on the
// int8 MFMA: the GEMM reads copies of A and B with every byte's top bit
// flipped, i.e. the signed byte u - 128, and since
//   sum_k u_a u_b = sum_k (u_a - 128)(u_b - 128) + 128 (sum_k u_a + sum_k u_b) - 16384 K,
// each output's accumulator starts at 128 times the sum along K of its A row
// and B column, minus 16384 K (int32 arithmetic wraps, so the result is
// exact whenever it fits).  These kernels write the flipped copies and the
// sums in one pass over each operand: sums[l][r] = sum_k X[l][r][k] for a
// K-major operand (r = m or n), or sum_k X[l][k][r] for an M-major A /
// N-major B.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_epi_prep.hpp"

namespace gemm_epi {

namespace {

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

constexpr unsigned kFlip = 0x80808080u;

// Sum of the four bytes of each word, added to acc.
__device__ __forceinline__ unsigned bytesum(v4u_t w, unsigned acc) {
  acc = __builtin_amdgcn_udot4(w.x, 0x01010101u, acc, false);
  acc = __builtin_amdgcn_udot4(w.y, 0x01010101u, acc, false);
  acc = __builtin_amdgcn_udot4(w.z, 0x01010101u, acc, false);
  return __builtin_amdgcn_udot4(w.w, 0x01010101u, acc, false);
}

// K-major: one wave per row, 16 bytes per lane and step (K bytes per row are
// a multiple of 16), then a sum across the wave.
__global__ __launch_bounds__(256) void prep_kmajor(const uint8_t* x, int64_t rows, int64_t K, uint8_t* flipped,
                                                   int32_t* sums) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // over L * R rows
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const v4u_t* p = (const v4u_t*)(x + row * K);
  v4u_t* q = (v4u_t*)(flipped + row * K);
  unsigned acc = 0;
  for (int64_t c = lane; c < K / 16; c += 64) {
    const v4u_t w = __builtin_nontemporal_load(p + c);
    q[c] = w ^ kFlip;
    acc = bytesum(w, acc);
  }
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) sums[row] = (int32_t)acc;
}

// M-major A / N-major B: a block covers 256 consecutive r (16 groups of 16)
// and a chunk of kchunk k-rows; thread t owns the 16 r of group t % 16 and
// every 16th k-row of the chunk from t / 16 on (a wave reads four k-rows of
// 256 contiguous bytes).  The 16 partial sums per r are added through LDS,
// and one atomic per r and block adds the chunk's sum into sums (zeroed
// first).
constexpr int kMnChunk = 512;
__global__ __launch_bounds__(256) void prep_mnmajor(const uint8_t* x, int64_t R, int64_t K, uint8_t* flipped,
                                                    int32_t* sums) {
  __shared__ unsigned part[16][16][17];  // [k-lane][r group][r in group], padded
  const int t = threadIdx.x, grp = t % 16, kl = t / 16;
  const int64_t r16 = (int64_t)blockIdx.x * 16 + grp;  // group of 16 r
  const int l = blockIdx.z;
  const bool live = r16 * 16 < R;
  const int64_t k0 = (int64_t)blockIdx.y * kMnChunk;
  const int64_t k1 = k0 + kMnChunk < K ? k0 + kMnChunk : K;
  const int64_t base = (int64_t)l * K * R + r16 * 16;
  unsigned s[16] = {};
  if (live) {
#pragma unroll 8
    for (int64_t k = k0 + kl; k < k1; k += 16) {
      const v4u_t w = __builtin_nontemporal_load((const v4u_t*)(x + base + k * R));
      *(v4u_t*)(flipped + base + k * R) = w ^ kFlip;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned v = w[j];
        s[4 * j + 0] += v & 0xff;
        s[4 * j + 1] += (v >> 8) & 0xff;
        s[4 * j + 2] += (v >> 16) & 0xff;
        s[4 * j + 3] += v >> 24;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) part[kl][grp][j] = s[j];
  __syncthreads();
  // thread t adds up r = 16 * (t / 16) + t % 16 of this block over the k-lanes
  const int g2 = t / 16, j2 = t % 16;
  unsigned sum = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) sum += part[k][g2][j2];
  const int64_t r = ((int64_t)blockIdx.x * 16 + g2) * 16 + j2;
  if (r < R) atomicAdd(sums + (int64_t)l * R + r, (int32_t)sum);
}

// fp8 -> fp16, 16 elements per thread and step.  Every finite e4m3 and e5m2
// value, subnormals included, is an fp16 value (e4m3: |v| <= 448, steps down
// to 2^-9; e5m2: |v| <= 57344, steps down to 2^-16), so the conversion with a
// scale of 1 is exact, and NaN stays NaN.
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
template <bool E5M2>
__device__ __forceinline__ unsigned widen2(unsigned w, bool hi) {
  v2h_t h;
  if constexpr (E5M2)
    h = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true) : __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false);
  else
    h = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(unsigned, h);
}
template <bool E5M2>
__global__ __launch_bounds__(256) void widen_f8(const uint8_t* x, int64_t groups, uint16_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += stride) {
    const v4u_t w = __builtin_nontemporal_load((const v4u_t*)x + g);
    v4u_t lo, hi;
    lo.x = widen2<E5M2>(w.x, false);
    lo.y = widen2<E5M2>(w.x, true);
    lo.z = widen2<E5M2>(w.y, false);
    lo.w = widen2<E5M2>(w.y, true);
    hi.x = widen2<E5M2>(w.z, false);
    hi.y = widen2<E5M2>(w.z, true);
    hi.z = widen2<E5M2>(w.w, false);
    hi.w = widen2<E5M2>(w.w, true);
    ((v4u_t*)out)[2 * g] = lo;
    ((v4u_t*)out)[2 * g + 1] = hi;
  }
}

__global__ __launch_bounds__(256) void fill_zero(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace

void launch_f8_widen(const uint8_t* x, int64_t n, bool e5m2, uint16_t* out, hipStream_t s) {
  const int64_t groups = n / 16;
  const int64_t blocks = (groups + 255) / 256;
  const dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192));
  if (e5m2)
    hipLaunchKernelGGL(widen_f8<true>, grid, dim3(256), 0, s, x, groups, out);
  else
    hipLaunchKernelGGL(widen_f8<false>, grid, dim3(256), 0, s, x, groups, out);
}

void launch_u8_prep(const uint8_t* x, bool kmajor, int64_t L, int64_t R, int64_t K, uint8_t* flipped,
                    int32_t* sums, hipStream_t s) {
  if (kmajor) {
    const int64_t rows = L * R;
    hipLaunchKernelGGL(prep_kmajor, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, rows, K, flipped, sums);
  } else {
    const int64_t n = L * R;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                       s, sums, n);
    const dim3 grid((unsigned)((R + 255) / 256), (unsigned)((K + kMnChunk - 1) / kMnChunk), (unsigned)L);
    hipLaunchKernelGGL(prep_mnmajor, grid, dim3(256), 0, s, x, R, K, flipped, sums);
  }
}

}  // namespace gemm_epi
