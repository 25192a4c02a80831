// gemm_epi_splitk.hip -- the second kernel of a split-K launch: adds the K
// slices' partial sums and applies the fused epilogue.
//
// With split K, slice s of the GEMM writes its fp32 (int32 for int8 inputs)
// partial accumulator for every output to ws + s * L*M*N, in D's layout.  The
// accumulator of an output is the sum of its slices (fp32 sums in slice
// order; int32 sums wrap, so they are exact whenever the result fits), and
// the epilogue is the one the GEMM kernel applies otherwise (CuTe DSL
// example custom_epilogue_dense_gemm.py, module docstring and its epilogue
// function):
//   Y = acc,  D = alpha*acc + beta*C + x_factor*X   (or the clamped form)
// C, X, D, Y and ws share one packed layout, so output element i of every
// array is element i of the flat range.  Each thread takes four consecutive
// elements: 16 bytes of every slice, 8 or 16 bytes of C, X, D, Y.  The flat
// length is a multiple of 4 (the 16-byte rule on the contiguous extent).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_epi_splitk.hpp"

namespace gemm_epi {

namespace {

typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef _Float16 v4h_t __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));

// Raw bits of four elements of type dt at element index i (16 bytes of a
// 4-byte type, 8 of a 2-byte type in .xy).
__device__ __forceinline__ v4u_t ld4(const void* base, int dt, int64_t i) {
  if (dt == SK_F32 || dt == SK_I32) return __builtin_nontemporal_load((const v4u_t*)((const uint32_t*)base + i));
  const v2u_t u = __builtin_nontemporal_load((const v2u_t*)((const uint16_t*)base + i));
  return v4u_t{u.x, u.y, 0u, 0u};
}

__device__ __forceinline__ v4f_t decode4(v4u_t r, int dt) {
  if (dt == SK_F32) return __builtin_bit_cast(v4f_t, r);
  if (dt == SK_BF16)
    return v4f_t{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                 __uint_as_float(r.y & 0xffff0000u)};
  const v4h_t h = __builtin_bit_cast(v4h_t, v2u_t{r.x, r.y});
  return v4f_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
}

// Round to nearest-even into type dt and store four elements at index i.
__device__ __forceinline__ void st4(void* base, int dt, int64_t i, v4f_t v) {
  if (dt == SK_F16) {
    const v4h_t h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    __builtin_nontemporal_store(__builtin_bit_cast(v2u_t, h), (v2u_t*)((uint16_t*)base + i));
  } else if (dt == SK_BF16) {
    const v4bf_t b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    __builtin_nontemporal_store(__builtin_bit_cast(v2u_t, b), (v2u_t*)((uint16_t*)base + i));
  } else {
    __builtin_nontemporal_store(v, (v4f_t*)((float*)base + i));
  }
}

__global__ __launch_bounds__(256) void splitk_epilogue_kernel(SplitkParams p) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < p.groups; g += stride) {
    const int64_t i = g * 4;
    if (p.int_path) {
      v4u_t a = __builtin_nontemporal_load((const v4u_t*)p.ws + g);
      for (int s = 1; s < p.splits; ++s) a += __builtin_nontemporal_load((const v4u_t*)p.ws + s * p.groups + g);
      v4u_t t = a * (unsigned)p.ialpha;
      if (p.C) t += ld4(p.C, SK_I32, i) * (unsigned)p.ibeta;
      if (p.relu)
        t = v4u_t{(int)t.x > 0 ? t.x : 0u, (int)t.y > 0 ? t.y : 0u, (int)t.z > 0 ? t.z : 0u,
                  (int)t.w > 0 ? t.w : 0u};
      if (p.X) t += ld4(p.X, SK_I32, i) * (unsigned)p.ix;
      __builtin_nontemporal_store(t, (v4u_t*)p.D + g);
      if (p.Y) __builtin_nontemporal_store(a, (v4u_t*)p.Y + g);
    } else {
      v4f_t a = __builtin_nontemporal_load((const v4f_t*)p.ws + g);
      for (int s = 1; s < p.splits; ++s) a += __builtin_nontemporal_load((const v4f_t*)p.ws + s * p.groups + g);
      // D = alpha * acc + beta * C (clamped at 0 in the ReLU form) + x_factor * X
      v4f_t t = a * p.alpha;
      if (p.C) {
        const v4f_t c = decode4(ld4(p.C, p.c_dtype, i), p.c_dtype);
        t.x = __builtin_fmaf(p.beta, c.x, t.x);
        t.y = __builtin_fmaf(p.beta, c.y, t.y);
        t.z = __builtin_fmaf(p.beta, c.z, t.z);
        t.w = __builtin_fmaf(p.beta, c.w, t.w);
      }
      if (p.relu)
        t = v4f_t{t.x > 0.0f ? t.x : 0.0f, t.y > 0.0f ? t.y : 0.0f, t.z > 0.0f ? t.z : 0.0f,
                  t.w > 0.0f ? t.w : 0.0f};
      if (p.X) {
        const v4f_t x = decode4(ld4(p.X, p.x_dtype, i), p.x_dtype);
        t.x = __builtin_fmaf(p.xf, x.x, t.x);
        t.y = __builtin_fmaf(p.xf, x.y, t.y);
        t.z = __builtin_fmaf(p.xf, x.z, t.z);
        t.w = __builtin_fmaf(p.xf, x.w, t.w);
      }
      st4(p.D, p.d_dtype, i, t);
      if (p.Y) st4(p.Y, p.y_dtype, i, a);
    }
  }
}

}  // namespace

void launch_splitk_epilogue(const SplitkParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(splitk_epilogue_kernel, dim3(grid), dim3(256), 0, s, p);
}

}  // namespace gemm_epi
