// mfma_ceiling.hip -- measurement tool (not part of the GEMM path): the
// steady shader clock and throughput of a register-only MFMA stream on one
// workgroup per CU, with constant or with random operands, for the
// instructions the GEMM kernels use (fp16, bf16, int8, fp8 e4m3; 32x32 or
// 16x16 blocks).  Under the board power cap the clock, and so the attainable
// MFMA rate, depends on how many operand bits toggle; the GEMM's fraction of
// this rate, measured on data of its own distribution, separates its own
// losses from the part's power limit.
//
// Each wave keeps 8 operand fragments of 16 bytes and 8 independent 32x32
// accumulators (16 for 16x16 blocks, two instructions per 32x32 one); the
// fragments rotate every MFMA, so every instruction sees different operands
// (fp8 instructions take 32 bytes: two neighbouring fragments).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <vector>

#include "mfma_ceiling.h"

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8, kFrag = 8, kAcc = 8, kUnroll = 8;

// Operand types: the public GEMM header's codes.
enum : int { T_F16 = 1, T_BF16 = 2, T_E4M3 = 3, T_I8 = 4 };

// FLOP (OP for int8) of one 32x32 step: one 32x32 instruction or two 16x16.
__host__ __device__ constexpr double step_flop(int type) {
  return type == T_I8 ? 2.0 * 32 * 32 * 32 : type == T_E4M3 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
}

template <int TYPE, int BLK>
struct Stream {
  static constexpr bool INT = TYPE == T_I8;
  typedef typename std::conditional<BLK == 32, typename std::conditional<INT, v16i, v16f>::type,
                                    typename std::conditional<INT, v4i, v4f>::type>::type acc_t;
  __device__ static acc_t mma(const v4i& a0, const v4i& a1, const v4i& b0, const v4i& b1, const acc_t& c) {
    if constexpr (TYPE == T_F16) {
      const v8h a = __builtin_bit_cast(v8h, a0), b = __builtin_bit_cast(v8h, b0);
      if constexpr (BLK == 32) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
      else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    } else if constexpr (TYPE == T_BF16) {
      const v8bf a = __builtin_bit_cast(v8bf, a0), b = __builtin_bit_cast(v8bf, b0);
      if constexpr (BLK == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
      else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    } else if constexpr (TYPE == T_I8) {
      if constexpr (BLK == 32) return __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, c, 0, 0, 0);
      else return __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, c, 0, 0, 0);
    } else {
      const v8i a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      const v8i b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      if constexpr (BLK == 32) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
      else return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
  }
};

template <int TYPE, int BLK>
__global__ __launch_bounds__(kWaves * 64, 1) void mfma_stream(const v4i* src, float* out, long long* clk,
                                                              int iters) {
  using ST = Stream<TYPE, BLK>;
  using acc_t = typename ST::acc_t;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  v4i f[kFrag];
#pragma unroll
  for (int i = 0; i < kFrag; ++i) f[i] = src[(wave * kFrag + i) * 64 + lane];
  constexpr int NACC = BLK == 32 ? kAcc : 2 * kAcc;
  acc_t acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = acc_t{};
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; it += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        acc[i] = ST::mma(f[(i + u) % kFrag], f[(i + u + 1) % kFrag], f[(i + 3 + 2 * u) % kFrag],
                         f[(i + 4 + 2 * u) % kFrag], acc[i]);
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NACC; ++i) s += (float)acc[i][lane & 3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = w1 - w0;  // wall clock ticks at 100 MHz
  }
}

template <int TYPE>
void launch(int block, int blocks, const v4i* src, float* out, long long* clk, int iters) {
  if (block == 32)
    hipLaunchKernelGGL((mfma_stream<TYPE, 32>), dim3(blocks), dim3(kWaves * 64), 0, 0, src, out, clk, iters);
  else
    hipLaunchKernelGGL((mfma_stream<TYPE, 16>), dim3(blocks), dim3(kWaves * 64), 0, 0, src, out, clk, iters);
}

// One random 16-bit operand element from 16 random bits r (fp16, bf16):
// uniform sign, exponent 2^-1 .. 2^-4 (the magnitudes of a uniform (-1, 1)
// draw) and mantissa.
uint32_t random_half(int type, uint32_t r) {
  if (type == T_BF16) return (r & 0x8000u) | ((123u + ((r >> 7) & 3)) << 7) | (r & 0x7Fu);
  return (r & 0x8000u) | ((11u + ((r >> 10) & 3)) << 10) | (r & 0x3FFu);
}

// One random byte operand from 8 random bits r: int8 uniform over all 256
// values; e4m3 uniform sign, exponent field 0..8 and mantissa (|v| < 4,
// subnormals included, no NaN code).
uint32_t random_byte(int type, uint32_t r) {
  if (type == T_I8) return r & 0xFFu;
  return (r & 0x80u) | (((r >> 8) % 9u) << 3) | (r & 7u);
}

}  // namespace

extern "C" int mfma_ceiling_run_type(int type, int block, int random_operands, int iters, int reps, float* ms_out,
                                     double* ghz_out, double* tflops_out) {
  if (block != 32 && block != 16) return (int)hipErrorInvalidValue;
  if (type != T_F16 && type != T_BF16 && type != T_E4M3 && type != T_I8) return (int)hipErrorInvalidValue;
  int dev = 0;
  hipDeviceProp_t prop;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return (int)e;
  const int blocks = prop.multiProcessorCount;
  iters = (iters / kUnroll) * kUnroll;
  const size_t nfrag = (size_t)blocks * kWaves * kFrag * 64;
  std::vector<v4i> host(nfrag);
  uint64_t x = 0x9E3779B97F4A7C15ull;  // xorshift64 state
  auto next = [&]() {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
  };
  const bool bytes = type == T_I8 || type == T_E4M3;
  const uint32_t one = type == T_F16 ? 0x3C003C00u : type == T_BF16 ? 0x3F803F80u : type == T_I8 ? 0x01010101u
                                                                                                  : 0x38383838u;
  for (size_t i = 0; i < nfrag; ++i)
    for (int j = 0; j < 4; ++j) {
      uint32_t w = one;  // every element 1 (1.0)
      if (random_operands) {
        const uint64_t r = next();
        if (bytes)
          w = random_byte(type, (uint32_t)r) | random_byte(type, (uint32_t)(r >> 16)) << 8 |
              random_byte(type, (uint32_t)(r >> 32)) << 16 | random_byte(type, (uint32_t)(r >> 48)) << 24;
        else
          w = random_half(type, (uint32_t)(r >> 8)) | random_half(type, (uint32_t)(r >> 40)) << 16;
      }
      host[i][j] = (int)w;
    }
  v4i* src = nullptr;
  float* out = nullptr;
  long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.0f;
  long long c[2] = {0, 0};
  e = hipMalloc((void**)&src, nfrag * sizeof(v4i));
  if (e == hipSuccess) e = hipMalloc((void**)&out, (size_t)blocks * kWaves * 64 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc((void**)&clk, (size_t)blocks * 2 * sizeof(long long));
  if (e == hipSuccess) e = hipMemcpy(src, host.data(), nfrag * sizeof(v4i), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  for (int r = 0; e == hipSuccess && r <= reps; ++r) {
    e = hipEventRecord(e0, 0);
    const int n = r == 0 ? kUnroll * 64 : iters;
    switch (type) {
      case T_F16: launch<T_F16>(block, blocks, src, out, clk, n); break;
      case T_BF16: launch<T_BF16>(block, blocks, src, out, clk, n); break;
      case T_I8: launch<T_I8>(block, blocks, src, out, clk, n); break;
      default: launch<T_E4M3>(block, blocks, src, out, clk, n); break;
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  }
  if (e == hipSuccess) e = hipMemcpy(c, clk, sizeof c, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(src);
  (void)hipFree(out);
  (void)hipFree(clk);
  if (e != hipSuccess) return (int)e;
  const double flop = step_flop(type) * (double)iters * kAcc * kWaves * blocks;
  *ms_out = ms;
  *ghz_out = c[1] ? (double)c[0] / ((double)c[1] / 1e8) / 1e9 : 0.0;
  *tflops_out = flop / (ms * 1e-3) / 1e12;
  return 0;
}

extern "C" int mfma_ceiling_run(int block, int random_operands, int iters, int reps, float* ms_out, double* ghz_out,
                                double* tflops_out) {
  return mfma_ceiling_run_type(T_F16, block, random_operands, iters, reps, ms_out, ghz_out, tflops_out);
}
