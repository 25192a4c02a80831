/*
 * A plain C client of the C ABI (include/gemm_epi.h): no Python, no torch.
 * It allocates device memory with the HIP runtime's C API, runs two fused
 * GEMMs whose results have a closed form, and checks every output element.
 *
 *   fp16:  A = I (K = M, K-major), B integer-valued, C integer-valued:
 *          Y[m][n] = B[n][m] and D = 2*B^T + 3*C, all exact in fp16.
 *   int8:  A = I, B in [-128, 127], C in [-1000, 1000]:
 *          D = B^T - C exactly in int32.
 *
 * Exit status: 0 all checks passed, 1 a check failed, 77 no usable GPU.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gemm_epi.h"

#define N_ 256

static uint16_t f16_of_int(int v) { /* exact for |v| <= 2048 */
  if (v == 0) return 0;
  uint16_t sign = v < 0 ? 0x8000u : 0;
  unsigned a = (unsigned)(v < 0 ? -v : v);
  int e = 0;
  while ((a >> e) > 1) ++e;                  /* a = 1.f * 2^e */
  unsigned frac = (a << (10 - e)) & 0x3ffu;  /* e <= 10 */
  return (uint16_t)(sign | ((unsigned)(e + 15) << 10) | frac);
}

static int int_of_f16(uint16_t h) { /* integer-valued fp16 of magnitude < 2^11 */
  int e = (h >> 10) & 0x1f, f = h & 0x3ff;
  if (e == 0 && f == 0) return 0;
  int v = (1024 + f) >> (25 - e);
  return (h & 0x8000u) ? -v : v;
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
  if (host && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int check(int rc, const char* what) {
  if (rc != GEMM_EPI_OK) {
    fprintf(stderr, "%s: %s (%s)\n", what, gemm_epi_status_string(rc), gemm_epi_last_error());
    return 1;
  }
  return 0;
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    printf("c abi client: no GPU\n");
    return 77;
  }
  const size_t nn = (size_t)N_ * N_;
  uint16_t *a16 = calloc(nn, 2), *b16 = malloc(nn * 2), *c16 = malloc(nn * 2), *d16 = malloc(nn * 2),
           *y16 = malloc(nn * 2);
  int8_t *a8 = calloc(nn, 1), *b8 = malloc(nn);
  int32_t *c32 = malloc(nn * 4), *d32 = malloc(nn * 4);
  unsigned s = 12345u;
  for (size_t i = 0; i < nn; ++i) {
    s = s * 1103515245u + 12345u;
    b16[i] = f16_of_int((int)((s >> 16) % 9) - 4);
    c16[i] = f16_of_int((int)((s >> 8) % 7) - 3);
    b8[i] = (int8_t)(int)((s >> 12) & 0xff);
    c32[i] = (int32_t)((s >> 4) % 2001) - 1000;
  }
  for (int m = 0; m < N_; ++m) {
    a16[(size_t)m * N_ + m] = f16_of_int(1);
    a8[(size_t)m * N_ + m] = 1;
  }

  int bad = 0;
  gemm_epi_handle* h = NULL;
  /* fp16 */
  gemm_epi_desc d;
  memset(&d, 0, sizeof d);
  d.M = d.N = d.K = N_;
  d.L = 1;
  d.a_major = GEMM_EPI_MAJOR_K;
  d.b_major = GEMM_EPI_MAJOR_K;
  d.cd_major = GEMM_EPI_MAJOR_N;
  d.ab_dtype = GEMM_EPI_F16;
  d.c_dtype = GEMM_EPI_F16;
  d.d_dtype = GEMM_EPI_F16;
  d.y_dtype = GEMM_EPI_F16;
  d.epilogue = GEMM_EPI_LINEAR;
  void *dA = dev_copy(a16, nn * 2), *dB = dev_copy(b16, nn * 2), *dC = dev_copy(c16, nn * 2);
  void *dD = dev_copy(NULL, nn * 2), *dY = dev_copy(NULL, nn * 2);
  if (!dA || !dB || !dC || !dD || !dY) {
    printf("c abi client: device allocation failed\n");
    return 77;
  }
  if (check(gemm_epi_create(&d, &h), "create f16") ||
      check(gemm_epi_run(h, dA, dB, dC, NULL, dD, dY, 2.0f, 3.0f, 0.0f, NULL), "run f16"))
    return 1;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(d16, dD, nn * 2, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(y16, dY, nn * 2, hipMemcpyDeviceToHost) != hipSuccess)
    return 1;
  for (int m = 0; m < N_; ++m)
    for (int n = 0; n < N_; ++n) {
      const int bt = int_of_f16(b16[(size_t)n * N_ + m]), c = int_of_f16(c16[(size_t)m * N_ + n]);
      if (int_of_f16(y16[(size_t)m * N_ + n]) != bt || int_of_f16(d16[(size_t)m * N_ + n]) != 2 * bt + 3 * c) {
        if (bad++ < 5) fprintf(stderr, "f16 mismatch at (%d, %d)\n", m, n);
      }
    }
  gemm_epi_destroy(h);

  /* int8 */
  d.ab_dtype = GEMM_EPI_I8;
  d.c_dtype = GEMM_EPI_I32;
  d.d_dtype = GEMM_EPI_I32;
  d.y_dtype = GEMM_EPI_NONE;
  void *eA = dev_copy(a8, nn), *eB = dev_copy(b8, nn), *eC = dev_copy(c32, nn * 4), *eD = dev_copy(NULL, nn * 4);
  if (!eA || !eB || !eC || !eD) return 77;
  if (check(gemm_epi_create(&d, &h), "create int8") ||
      check(gemm_epi_run(h, eA, eB, eC, NULL, eD, NULL, 1.0f, -1.0f, 0.0f, NULL), "run int8"))
    return 1;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(d32, eD, nn * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return 1;
  for (int m = 0; m < N_; ++m)
    for (int n = 0; n < N_; ++n)
      if (d32[(size_t)m * N_ + n] != (int32_t)b8[(size_t)n * N_ + m] - c32[(size_t)m * N_ + n]) {
        if (bad++ < 5) fprintf(stderr, "int8 mismatch at (%d, %d)\n", m, n);
      }
  gemm_epi_destroy(h);
  hipFree(dA), hipFree(dB), hipFree(dC), hipFree(dD), hipFree(dY);
  hipFree(eA), hipFree(eB), hipFree(eC), hipFree(eD);
  if (bad) {
    fprintf(stderr, "c abi client: %d mismatches\n", bad);
    return 1;
  }
  printf("c abi client: ok (fp16 and int8, %d x %d)\n", N_, N_);
  return 0;
}
