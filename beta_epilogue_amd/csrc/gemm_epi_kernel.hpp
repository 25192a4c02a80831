// gemm_epi_kernel.hpp -- persistent fused-epilogue batched GEMM for gfx950.
//
// Operation (CuTe DSL example "custom_epilogue_dense_gemm.py", module
// docstring, "Tensor dimensions" and its epilogue formula):
//   Y = A.B^T,  D = alpha*(A.B^T) + beta*C + x_factor*X,  per batch l.
//
// Structure of one workgroup (4 waves, one wave per SIMD):
//   * persistent tile loop: workgroup ids are remapped so that each of the 8
//     XCDs walks a contiguous run of tiles of a grouped raster, which keeps
//     the A row panels and B column panels of concurrently running tiles in
//     that XCD's L2 (the pages' persistent scheduler, "Device side" of the
//     Blackwell pipeline API card, made XCD-aware);
//   * global -> LDS staging: each LDS row holds 128 bytes of K of one tile
//     row, split into eight 16-byte chunks stored at chunk ^ swizzle(row) so
//     that the MFMA fragment reads hit distinct banks.  K-major operands go
//     straight to LDS with buffer_load_dwordx4 ... lds (the buffer's range
//     check turns rows past M/N and chunks past K into zeros); M-major int8
//     A is loaded to registers, transposed 8x8 bytes with v_perm and written
//     with ds_write_b64.  Two stages: the next K tile streams in while the
//     current one is multiplied (the pages' multi-stage pipeline, "Depth and
//     shared memory");
//   * MFMA mainloop: v_mfma_f32_32x32x16_{f16,bf16}, v_mfma_f32_32x32x64_f8f6f4
//     (e4m3 x e4m3) or v_mfma_i32_32x32x32_i8; each wave owns a 128x128
//     quarter of the 256x256 tile, 16 accumulator blocks of 32x32;
//   * fused epilogue on the fp32 (int32) accumulator: Y = acc, D = alpha*acc
//     + beta*C + x_factor*X, rounded to nearest-even into the output types;
//     all loads of an element precede its stores (the example's epilogue
//     comment), C and X are only read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

// Element type codes; the same numbers as the public header.
enum : int { T_NONE = 0, T_F16 = 1, T_BF16 = 2, T_E4M3 = 3, T_I8 = 4, T_F32 = 5, T_I32 = 6 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Kernel arguments (passed by value).
struct Params {
  const void* A;
  const void* B;
  const void* C;  // NULL when the beta term is skipped
  const void* X;  // NULL when the x_factor term is skipped
  void* D;
  void* Y;        // NULL when Y is not written
  int64_t M, N, K;
  int64_t tiles_total;
  int32_t L, tiles_m, tiles_n, group_m;
  int32_t c_dtype, x_dtype, d_dtype, y_dtype;  // T_NONE for skipped terms
  float alpha, beta, xf;
  int32_t ialpha, ibeta, ix;  // integral scalars for int32 outputs
  int32_t xcd_remap;          // grid is a multiple of 8: remap ids per XCD
};

// ---------------------------------------------------------------------------
// MFMA traits per A/B element type.  KSB = bytes of K one MFMA consumes per
// row; each lane holds half of them (lanes 32..63 take the upper half).  A
// and B fragments use the same lane -> k assignment, so the contraction is
// exact whatever order the matrix core walks k in.
// ---------------------------------------------------------------------------
template <int AB> struct Mma;

template <> struct Mma<T_F16> {
  typedef v16f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_BF16> {
  typedef v16f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_I8> {
  typedef v16i acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 1, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<T_E4M3> {
  typedef v16f acc_t;
  typedef v8i frag_t;
  static constexpr int ESIZE = 1, KSB = 64;
  // Format selectors 0/0 = fp8 e4m3 for both operands; zero scale operands
  // select the unscaled instruction.
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// Compile-time kernel configuration.
template <int AB_, bool A_KMAJOR_, bool B_KMAJOR_, bool CD_NMAJOR_>
struct Cfg {
  static constexpr int AB = AB_;
  static constexpr bool A_KMAJOR = A_KMAJOR_, B_KMAJOR = B_KMAJOR_, CD_NMAJOR = CD_NMAJOR_;
  static constexpr int BM = 256, BN = 256;           // workgroup tile
  static constexpr int ROWB = 128;                   // K bytes per LDS row per stage
  static constexpr int BK = ROWB / Mma<AB>::ESIZE;   // K elements per stage
  static constexpr int WAVES_M = 2, WAVES_N = 2;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = NW * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;           // 32x32 blocks
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int STAGES = 2;
  static constexpr int PIPE_BYTES = STAGES * STAGE_BYTES;
  static constexpr int EPI_BYTES = NW * 64 * 132 * 4;  // per-wave epilogue regions
  static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  static constexpr int KSTEPS = ROWB / Mma<AB>::KSB;
};

// Chunk swizzle: the 16-byte chunk c of LDS row r lives at c ^ swz(r).
__device__ __forceinline__ int swz(int row) { return row & 7; }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------
// Staging of a K-major operand tile (R rows x 128 bytes) straight into LDS.
// One wave instruction moves 64 chunks = 8 rows = 1 KiB of LDS, written
// linearly: lane j fills physical chunk j%8 of row j/8, so it fetches the
// logical chunk (j%8) ^ swz(row) from global memory.
// ---------------------------------------------------------------------------
template <int R, int NW>
struct KMajorStager {
  static constexpr int NQ = R / (8 * NW);
  static_assert(NQ * 8 * NW == R, "rows must split evenly over the waves");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[NQ];
  uint32_t cbyte;  // byte offset of this lane's logical chunk within a row

  __device__ __forceinline__ void setup(const char* tile_base, int64_t ld_bytes, int valid_rows,
                                        int wave, int lane) {
    const int rsub = lane >> 3;
    const int c = (lane & 7) ^ (rsub & 7);
    cbyte = (uint32_t)c * 16u;
    const uint32_t nrec = (uint32_t)((int64_t)valid_rows * ld_bytes);
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)tile_base, (short)0, (int)nrec, 0x00020000);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int row = (q * NW + wave) * 8 + rsub;
      voff[q] = (uint32_t)(row * ld_bytes) + cbyte;
    }
  }

  // Issue the loads of K tile kt into the LDS region at byte offset lds_off.
  // kvalid = bytes of K left from this K tile on (chunks at or past it read 0).
  __device__ __forceinline__ void issue(char* lds, int lds_off, int wave, int kt, int64_t kvalid) {
    const uint32_t kofs = (uint32_t)kt * 128u;
    const bool live = (int64_t)cbyte < kvalid;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t vo = live ? voff[q] + kofs : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void_t*)(lds + lds_off + (q * NW + wave) * 1024), 16, vo, 0, 0, 0);
    }
  }
};

// 4x4 byte transpose: x_r holds bytes (r,0..3); c_j receives bytes (0..3, j).
__device__ __forceinline__ void tr4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                      uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3) {
  const uint32_t u0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
  const uint32_t u1 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
  const uint32_t v0 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t v1 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  c0 = __builtin_amdgcn_perm(v0, u0, 0x05040100u);
  c1 = __builtin_amdgcn_perm(v0, u0, 0x07060302u);
  c2 = __builtin_amdgcn_perm(v1, u1, 0x05040100u);
  c3 = __builtin_amdgcn_perm(v1, u1, 0x07060302u);
}

// ---------------------------------------------------------------------------
// Staging of an M-major one-byte A tile: global A[l][k][m], 128 k rows by
// BM m bytes per stage.  Each thread owns blocks of 8 k x 8 m bytes: eight
// 8-byte global loads (a wave covers whole 256-byte k rows), an 8x8 byte
// transpose in registers, then eight 8-byte LDS writes into the same
// K-contiguous swizzled layout the K-major path produces.
// ---------------------------------------------------------------------------
template <int BM, int THREADS>
struct MMajorStager8 {
  static constexpr int MB = BM / 8;                 // m blocks per tile
  static constexpr int NB = (128 / 8) * MB / THREADS;  // blocks per thread
  static_assert(NB * THREADS == 16 * MB, "blocks must split evenly");
  uint2 buf[NB][8];
  const char* base;  // A + l*M*K (bytes)
  int64_t M, K;
  int m0;

  __device__ __forceinline__ void setup(const char* a_batch, int64_t M_, int64_t K_, int m0_) {
    base = a_batch;
    M = M_;
    K = K_;
    m0 = m0_;
  }

  __device__ __forceinline__ void load(int kt, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = b * THREADS + tid;
      const int bm = id % MB, bk = id / MB;
      const int64_t m = (int64_t)m0 + bm * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = (int64_t)kt * 128 + bk * 8 + r;
        if (k < K && m < M)
          buf[b][r] = *(const uint2*)(base + k * M + m);
        else
          buf[b][r] = make_uint2(0u, 0u);
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int lds_off, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = b * THREADS + tid;
      const int bm = id % MB, bk = id / MB;
      uint32_t lo[8], hi[8];
      tr4x4(buf[b][0].x, buf[b][1].x, buf[b][2].x, buf[b][3].x, lo[0], lo[1], lo[2], lo[3]);
      tr4x4(buf[b][4].x, buf[b][5].x, buf[b][6].x, buf[b][7].x, hi[0], hi[1], hi[2], hi[3]);
      tr4x4(buf[b][0].y, buf[b][1].y, buf[b][2].y, buf[b][3].y, lo[4], lo[5], lo[6], lo[7]);
      tr4x4(buf[b][4].y, buf[b][5].y, buf[b][6].y, buf[b][7].y, hi[4], hi[5], hi[6], hi[7]);
      const int chunk = bk >> 1, sub = (bk & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = bm * 8 + i;
        const int off = lds_off + row * 128 + ((chunk ^ swz(row)) << 4) + sub;
        *(uint2*)(lds + off) = make_uint2(lo[i], hi[i]);
      }
    }
  }
};

// Fragment read: this lane's half of k step s of LDS row `row`.
template <int AB>
__device__ __forceinline__ typename Mma<AB>::frag_t read_frag(const char* lds, int tile_off, int row,
                                                              int s, int half) {
  constexpr int KSB = Mma<AB>::KSB;
  if constexpr (KSB == 32) {
    const int c = s * 2 + half;
    return *(const v4i*)(lds + tile_off + row * 128 + ((c ^ swz(row)) << 4));
  } else {
    const int c = s * 4 + half * 2;
    const v4i lo = *(const v4i*)(lds + tile_off + row * 128 + ((c ^ swz(row)) << 4));
    const v4i hi = *(const v4i*)(lds + tile_off + row * 128 + (((c + 1) ^ swz(row)) << 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// ---------------------------------------------------------------------------
// Fused epilogue (on the accumulator of one wave: rows [mw, mw+WM), columns
// [nw, nw+WN) of batch l).  Y = acc; D = alpha*acc + beta*C + x_factor*X in
// fp32 (int32, wrapping, for int8 inputs), rounded to nearest-even into the
// output type; every load of an element precedes its stores.
// ---------------------------------------------------------------------------
template <class CF>
struct EpiLayout {
  static constexpr int LINES = 64;        // lines per half
  static constexpr int LINE = 128;        // contiguous elements per line
  static constexpr int PITCH = LINE + 4;  // words per line in LDS
  static constexpr int WAVE_BYTES = LINES * PITCH * 4;
  static constexpr int BYTES = CF::NW * WAVE_BYTES;
};

__device__ __forceinline__ v4f load4_f(const void* p, int dt, int64_t i) {
  if (dt == T_F16) {
    const v2u u = __builtin_nontemporal_load((const v2u*)((const _Float16*)p + i));
    const _Float16* h = (const _Float16*)&u;
    return v4f{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
  if (dt == T_BF16) {
    const v2u u = __builtin_nontemporal_load((const v2u*)((const uint16_t*)p + i));
    return v4f{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  }
  return __builtin_nontemporal_load((const v4f*)((const float*)p + i));
}

__device__ __forceinline__ void store4_f(void* p, int dt, int64_t i, v4f v) {
  if (dt == T_F16) {
    _Float16 h[4] = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    __builtin_nontemporal_store(*(const v2u*)h, (v2u*)((_Float16*)p + i));
  } else if (dt == T_BF16) {
    __bf16 b[4] = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    __builtin_nontemporal_store(*(const v2u*)b, (v2u*)((uint16_t*)p + i));
  } else {
    __builtin_nontemporal_store(v, (v4f*)((float*)p + i));
  }
}

// Accumulator element as the 32-bit pattern stored in LDS.  (The element is
// read into a scalar first: bit-casting a vector-element lvalue directly
// reads element 0 with this compiler.)
__device__ __forceinline__ float acc_bits(float v) { return v; }
__device__ __forceinline__ float acc_bits(int v) { return __int_as_float(v); }

template <class CF, class ACC>
__device__ __forceinline__ void epilogue(const Params& p, const ACC (&acc)[CF::FM][CF::FN], char* lds,
                                         int wave, int lane, int l, int mw, int nw) {
  using EL = EpiLayout<CF>;
  constexpr bool NMAJ = CF::CD_NMAJOR;
  const int region = wave * EL::WAVE_BYTES;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t obase = (int64_t)l * p.M * p.N;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // -- scatter this half of the accumulator into the wave's LDS region.
    // N-major: lines are rows (i blocks 2h, 2h+1), elements are columns.
    // M-major: lines are columns (j blocks 2h, 2h+1), elements are rows.
    if constexpr (NMAJ) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < CF::FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int line = ii * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
            const int col = j * 32 + l32;
            const auto e = acc[2 * h + ii][j][v];
            *(float*)(lds + region + (line * EL::PITCH + col) * 4) = acc_bits(e);
          }
    } else {
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int line = jj * 32 + l32;
            const int row = i * 32 + v4 * 8 + half * 4;
            const ACC& a = acc[i][2 * h + jj];
            const auto e0 = a[v4 * 4 + 0], e1 = a[v4 * 4 + 1];
            const auto e2 = a[v4 * 4 + 2], e3 = a[v4 * 4 + 3];
            const v4f w = {acc_bits(e0), acc_bits(e1), acc_bits(e2), acc_bits(e3)};
            *(v4f*)(lds + region + (line * EL::PITCH + row) * 4) = w;
          }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // -- walk the half: lane reads 4 contiguous elements of line it*2+half.
    for (int it = 0; it < EL::LINES / 2; ++it) {
      const int line = it * 2 + half;
      const int e = l32 * 4;
      const v4f w = *(const v4f*)(lds + region + (line * EL::PITCH + e) * 4);
      int64_t m, n;
      if constexpr (NMAJ) {
        m = mw + h * 64 + line;
        n = nw + e;
      } else {
        n = nw + h * 64 + line;
        m = mw + e;
      }
      if (m < p.M && n < p.N) {
        const int64_t o = obase + (NMAJ ? m * p.N + n : n * p.M + m);
        if constexpr (CF::AB == T_I8) {
          const v4u a = __builtin_bit_cast(v4u, w);
          v4u t = a * (unsigned)p.ialpha;
          if (p.c_dtype) t += __builtin_nontemporal_load((const v4u*)((const int*)p.C + o)) * (unsigned)p.ibeta;
          if (p.x_dtype) t += __builtin_nontemporal_load((const v4u*)((const int*)p.X + o)) * (unsigned)p.ix;
          __builtin_nontemporal_store(t, (v4u*)((int*)p.D + o));
          if (p.y_dtype) __builtin_nontemporal_store(a, (v4u*)((int*)p.Y + o));
        } else {
          v4f t = w * p.alpha;
          if (p.c_dtype) {
            const v4f c = load4_f(p.C, p.c_dtype, o);
            t.x = __builtin_fmaf(p.beta, c.x, t.x);
            t.y = __builtin_fmaf(p.beta, c.y, t.y);
            t.z = __builtin_fmaf(p.beta, c.z, t.z);
            t.w = __builtin_fmaf(p.beta, c.w, t.w);
          }
          if (p.x_dtype) {
            const v4f x = load4_f(p.X, p.x_dtype, o);
            t.x = __builtin_fmaf(p.xf, x.x, t.x);
            t.y = __builtin_fmaf(p.xf, x.y, t.y);
            t.z = __builtin_fmaf(p.xf, x.z, t.z);
            t.w = __builtin_fmaf(p.xf, x.w, t.w);
          }
          store4_f(p.D, p.d_dtype, o, t);
          if (p.y_dtype) store4_f(p.Y, p.y_dtype, o, w);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <class CF>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_epi_kernel(Params p) {
  using MM = Mma<CF::AB>;
  using acc_t = typename MM::acc_t;
  constexpr int ES = MM::ESIZE;
  constexpr int BM = CF::BM, BN = CF::BN;
  __shared__ __attribute__((aligned(1024))) char lds[CF::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % CF::WAVES_M, wn = wave / CF::WAVES_M;
  const int half = lane >> 5, l32 = lane & 31;

  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int g = p.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  const int64_t kbytes = p.K * ES;
  const int KT = (int)((kbytes + CF::ROWB - 1) / CF::ROWB);
  const int64_t tiles_mn = (int64_t)p.tiles_m * p.tiles_n;

  for (int64_t t = g; t < p.tiles_total; t += G) {
    // ---- tile coordinates: grouped raster inside each batch -------------
    const int l = (int)(t / tiles_mn);
    const int64_t r = t - (int64_t)l * tiles_mn;
    const int64_t gsize = (int64_t)p.group_m * p.tiles_n;
    const int gid = (int)(r / gsize);
    const int first_m = gid * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int within = (int)(r - (int64_t)gid * gsize);
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- staging set-up --------------------------------------------------
    const char* Ab = (const char*)p.A + (int64_t)l * p.M * kbytes;
    const char* Bb = (const char*)p.B + (int64_t)l * p.N * kbytes;
    KMajorStager<BN, CF::NW> sb;
    sb.setup(Bb + (int64_t)n0 * kbytes, kbytes, (int)min((int64_t)BN, p.N - n0), wave, lane);
    KMajorStager<BM, CF::NW> sa_k;
    MMajorStager8<BM, CF::THREADS> sa_m;
    if constexpr (CF::A_KMAJOR)
      sa_k.setup(Ab + (int64_t)m0 * kbytes, kbytes, (int)min((int64_t)BM, p.M - m0), wave, lane);
    else
      sa_m.setup(Ab, p.M, p.K, m0);

    acc_t acc[CF::FM][CF::FN];
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) acc[i][j] = acc_t{};

    // ---- prologue: K tile 0 into stage 0 --------------------------------
    if constexpr (CF::A_KMAJOR) {
      sa_k.issue(lds, 0, wave, 0, kbytes);
    } else {
      sa_m.load(0, tid);
      sa_m.store(lds, 0, tid);
    }
    sb.issue(lds, BM * 128, wave, 0, kbytes);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- mainloop ---------------------------------------------------------
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = (kt & 1) * CF::STAGE_BYTES;
      const int nxt = ((kt + 1) & 1) * CF::STAGE_BYTES;
      const bool more = kt + 1 < KT;
      if (more) {
        const int64_t kv = kbytes - (int64_t)(kt + 1) * 128;
        if constexpr (CF::A_KMAJOR)
          sa_k.issue(lds, nxt, wave, kt + 1, kv);
        else
          sa_m.load(kt + 1, tid);
        sb.issue(lds, nxt + BM * 128, wave, kt + 1, kv);
      }
#pragma unroll
      for (int s = 0; s < CF::KSTEPS; ++s) {
        typename MM::frag_t fa[CF::FM], fb[CF::FN];
#pragma unroll
        for (int i = 0; i < CF::FM; ++i)
          fa[i] = read_frag<CF::AB>(lds, cur, wm * CF::WM + i * 32 + l32, s, half);
#pragma unroll
        for (int j = 0; j < CF::FN; ++j)
          fb[j] = read_frag<CF::AB>(lds, cur + BM * 128, wn * CF::WN + j * 32 + l32, s, half);
#pragma unroll
        for (int i = 0; i < CF::FM; ++i)
#pragma unroll
          for (int j = 0; j < CF::FN; ++j) acc[i][j] = MM::mma(fa[i], fb[j], acc[i][j]);
      }
      if constexpr (!CF::A_KMAJOR) {
        if (more) sa_m.store(lds, nxt, tid);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // ---- fused epilogue ---------------------------------------------------
    // Each wave re-lays its 128x128 accumulator quarter out through a private
    // LDS region, half at a time (64 lines of 128 contiguous elements, lines
    // padded to 132 words), then walks it with one 16-byte LDS read per lane:
    // 32 lanes cover one 128-element line, so C/X loads and D/Y stores move 4
    // contiguous elements per lane and whole lines per half-wave.
    epilogue<CF>(p, acc, lds, wave, lane, l, m0 + wm * CF::WM, n0 + wn * CF::WN);
    __syncthreads();  // LDS is reused by the next tile's prologue
  }
}

}  // namespace gemm_epi
