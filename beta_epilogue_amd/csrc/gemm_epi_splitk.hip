// gemm_epi_splitk.hip -- the second kernel of a split-K launch: adds the K
// slices' partial sums of the split tiles and applies the fused epilogue.
//
// Slice s of split tile dp_tiles + j wrote its fp32 (int32 for int8 inputs)
// partial accumulator to workspace slot s*tail_tiles + j: the tile's
// rows x cols part inside the matrix, packed in D's majorness.  The
// accumulator of an output is the sum of its slices (fp32 sums in slice
// order; int32 sums wrap, so they are exact whenever the result fits), and
// the epilogue is the one the GEMM kernel applies otherwise (CuTe DSL
// example custom_epilogue_dense_gemm.py, module docstring and its epilogue
// function):
//   Y = acc,  D = alpha*acc + beta*C + x_factor*X   (or the clamped form)
// Each thread takes four consecutive elements along the contiguous dimension:
// 16 bytes of every slice, 8 or 16 bytes of C, X, D, Y.  The contiguous
// extent is a multiple of 4 elements (the 16-byte rule) and tiles start at
// multiples of 4, so a group of four lies in the matrix or wholly outside.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_epi_raster.hpp"
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
  const int64_t per_tile = (int64_t)p.tile_m * p.tile_n / 4;  // groups of a slot
  const int64_t groups = (int64_t)p.tail_tiles * per_tile;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < groups; q += stride) {
    const int j = (int)(q / per_tile);
    const int g = (int)(q - (int64_t)j * per_tile);
    const TileRC tc = raster_tile(p.dp_tiles + j, p.tiles_m, p.tiles_n, p.group_m);
    const int64_t m0 = (int64_t)tc.tm * p.tile_m, n0 = (int64_t)tc.tn * p.tile_n;
    const int rows = (int)min(p.M - m0, (int64_t)p.tile_m), cols = (int)min(p.N - n0, (int64_t)p.tile_n);
    // line (a row if N-major, a column if M-major) and position along it
    const int along_len = p.cd_nmajor ? cols : rows, lines = p.cd_nmajor ? rows : cols;
    const int per_line = (p.cd_nmajor ? p.tile_n : p.tile_m) / 4;
    const int line = g / per_line, pos = (g - line * per_line) * 4;
    if (line >= lines || pos >= along_len) continue;
    const int64_t e = (int64_t)line * along_len + pos;  // element of the slot
    const int64_t i = (int64_t)tc.l * p.M * p.N +
                      (p.cd_nmajor ? (m0 + line) * p.N + n0 + pos : (n0 + line) * p.M + m0 + pos);
    const int64_t slot_elems = (int64_t)p.tile_m * p.tile_n;
    if (p.int_path) {
      const uint32_t* w = (const uint32_t*)p.ws + (int64_t)j * slot_elems + e;
      v4u_t a = __builtin_nontemporal_load((const v4u_t*)w);
      for (int s = 1; s < p.splits; ++s)
        a += __builtin_nontemporal_load((const v4u_t*)(w + (int64_t)s * p.tail_tiles * slot_elems));
      v4u_t t = a * (unsigned)p.ialpha;
      if (p.C) t += ld4(p.C, SK_I32, i) * (unsigned)p.ibeta;
      if (p.relu)
        t = v4u_t{(int)t.x > 0 ? t.x : 0u, (int)t.y > 0 ? t.y : 0u, (int)t.z > 0 ? t.z : 0u,
                  (int)t.w > 0 ? t.w : 0u};
      if (p.X) t += ld4(p.X, SK_I32, i) * (unsigned)p.ix;
      __builtin_nontemporal_store(t, (v4u_t*)((uint32_t*)p.D + i));
      if (p.Y) __builtin_nontemporal_store(a, (v4u_t*)((uint32_t*)p.Y + i));
    } else {
      const float* w = (const float*)p.ws + (int64_t)j * slot_elems + e;
      v4f_t a = __builtin_nontemporal_load((const v4f_t*)w);
      for (int s = 1; s < p.splits; ++s)
        a += __builtin_nontemporal_load((const v4f_t*)(w + (int64_t)s * p.tail_tiles * slot_elems));
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
