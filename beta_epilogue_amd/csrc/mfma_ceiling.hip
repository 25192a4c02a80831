// mfma_ceiling.hip -- measurement tool (not part of the GEMM path): the
// steady shader clock and throughput of a register-only stream of
// v_mfma_f32_32x32x16_f16 or v_mfma_f32_16x16x32_f16 on one workgroup per
// CU, with constant or random operands.  Under the board power cap the clock, and so the attainable MFMA
// rate, depends on how many operand bits toggle; the GEMM's fraction of this
// rate, measured on data of its own distribution, separates its own losses
// from the part's power limit.
//
// Each wave keeps 8 operand fragments and 8 independent 32x32 accumulators;
// the fragment pairs rotate every MFMA, so every instruction sees different
// operands.  Random operands: fp16 values uniform in sign, exponent
// 2^-1 .. 2^-4 and mantissa (the magnitude range of a uniform (-1, 1) draw).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <vector>

#include "mfma_ceiling.h"

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8, kFrag = 8, kAcc = 8, kUnroll = 8;

typedef float v4f __attribute__((ext_vector_type(4)));

// BLK 32: v_mfma_f32_32x32x16_f16 on kAcc accumulators; BLK 16:
// v_mfma_f32_16x16x32_f16 (half the FLOP per instruction) on 2 * kAcc
// accumulators, two instructions per 32x32x16 one, so both shapes do the
// same FLOP per iteration.
template <int BLK>
__global__ __launch_bounds__(kWaves * 64, 1) void mfma_stream(const v4i* src, float* out, long long* clk,
                                                              int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  v4i f[kFrag];
#pragma unroll
  for (int i = 0; i < kFrag; ++i) f[i] = src[(wave * kFrag + i) * 64 + lane];
  constexpr int NACC = BLK == 32 ? kAcc : 2 * kAcc;
  typedef typename std::conditional<BLK == 32, v16f, v4f>::type acc_t;
  acc_t acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = acc_t{};
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; it += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < NACC; ++i) {
        const v8h a = __builtin_bit_cast(v8h, f[(i + u) % kFrag]);
        const v8h b = __builtin_bit_cast(v8h, f[(i + 3 + 2 * u) % kFrag]);
        if constexpr (BLK == 32)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
        else
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[i], 0, 0, 0);
      }
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NACC; ++i) s += acc[i][lane & 3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = w1 - w0;  // wall clock ticks at 100 MHz
  }
}

}  // namespace

// Runs the stream of block size `block` (32 or 16) on one workgroup per CU
// of the current device: a warm-up
// launch, then `reps` timed launches of `iters` (a multiple of 8) MFMAs per
// accumulator.  Reports the last launch: milliseconds (HIP events), the
// shader clock of workgroup 0 in GHz (clock64 against the 100 MHz wall
// clock) and TFLOP/s.  Returns 0, or a HIP error code.
extern "C" int mfma_ceiling_run(int block, int random_operands, int iters, int reps, float* ms_out,
                                double* ghz_out, double* tflops_out) {
  if (block != 32 && block != 16) return (int)hipErrorInvalidValue;
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
  for (size_t i = 0; i < nfrag; ++i)
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0x3C003C00u;  // two fp16 1.0
      if (random_operands) {
        const uint64_t r = next();
        const uint32_t a = (uint32_t)(r & 0x8000) | ((11u + ((r >> 16) & 3)) << 10) | (uint32_t)((r >> 20) & 0x3FF);
        const uint32_t b = (uint32_t)((r >> 32) & 0x8000) | ((11u + ((r >> 48) & 3)) << 10) | (uint32_t)((r >> 52) & 0x3FF);
        w = a | (b << 16);
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
    if (block == 32)
      hipLaunchKernelGGL(mfma_stream<32>, dim3(blocks), dim3(kWaves * 64), 0, 0, src, out, clk,
                         r == 0 ? kUnroll * 64 : iters);
    else
      hipLaunchKernelGGL(mfma_stream<16>, dim3(blocks), dim3(kWaves * 64), 0, 0, src, out, clk,
                         r == 0 ? kUnroll * 64 : iters);
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
  const double flop = 2.0 * 32 * 32 * 16 * (double)iters * kAcc * kWaves * blocks;
  *ms_out = ms;
  *ghz_out = c[1] ? (double)c[0] / ((double)c[1] / 1e8) / 1e9 : 0.0;
  *tflops_out = flop / (ms * 1e-3) / 1e12;
  return 0;
}
