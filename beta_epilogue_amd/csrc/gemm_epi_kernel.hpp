// gemm_epi_kernel.hpp -- persistent fused-epilogue batched GEMM for gfx950.
//
// Operation (CuTe DSL example "custom_epilogue_dense_gemm.py", module
// docstring, "Tensor dimensions" and its epilogue formula):
//   Y = A.B^T,  D = alpha*(A.B^T) + beta*C + x_factor*X,  per batch l.
//
// Structure of one workgroup (a compile-time configuration, see Cfg):
//   * persistent tile loop: workgroup ids are remapped so that each of the 8
//     XCDs walks a contiguous run of tiles of a grouped raster, which keeps
//     the A row panels and B column panels of concurrently running tiles in
//     that XCD's L2 (the persistent tile loop of the Blackwell pipeline API
//     card, "Device side", made XCD-aware);
//   * global -> LDS staging into a STAGES-deep ring: each LDS row holds ROWB
//     bytes of K of one tile row as 16-byte chunks stored at chunk ^ swz(row)
//     so that the MFMA fragment reads of 16 consecutive rows hit 16 distinct
//     16-byte bank groups of the 64-bank LDS.  K-major operands go straight
//     to LDS with buffer_load_dwordx4 ... lds (the buffer's range check turns
//     rows past M/N and chunks past K into zeros); M-major int8 A is loaded
//     to registers, transposed 8x8 bytes with v_perm and written with
//     ds_write_b64.  Each K tile waits only for its own stage (counted
//     vmcnt), so STAGES-1 tiles stay in flight (the multi-stage pipeline of
//     the API card's "Depth and shared memory");
//   * MFMA mainloop: v_mfma_f32_32x32x16_{f16,bf16}, v_mfma_f32_32x32x64_f8f6f4
//     (e4m3 x e4m3) or v_mfma_i32_32x32x32_i8 on 32x32 accumulator blocks in
//     AGPRs; the fragments of k step s+1 are read while step s multiplies;
//   * fused epilogue on the fp32 (int32) accumulator: Y = acc, D = alpha*acc
//     + beta*C + x_factor*X, rounded to nearest-even into the output types;
//     each 32-wide block of the accumulator is re-laid out through a small
//     per-wave LDS region so C/X loads and D/Y stores move 4 contiguous
//     elements per lane; all loads of an element precede its stores (the
//     example's epilogue comment) and C and X are only read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

// Element type codes; the same numbers as the public header.
enum : int { T_NONE = 0, T_F16 = 1, T_BF16 = 2, T_E4M3 = 3, T_I8 = 4, T_F32 = 5, T_I32 = 6, T_E5M2 = 7 };
// Kernel A/B codes of the fp8 pairs (A's format x B's).
enum : int { T_E4M3_E5M2 = 8, T_E5M2_E4M3 = 9 };
// Kernel A/B codes of fp8 operands widened to fp16 before the f16 MFMA (A's
// format x B's), used when an fp32 output is asked for.
enum : int { T_W_E4M3 = 10, T_W_E5M2 = 11, T_W_E4M3_E5M2 = 12, T_W_E5M2_E4M3 = 13 };

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
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
  int32_t epi_kind;           // element type shared by every C/X/D/Y in use (0: mixed)
  int32_t relu;               // D = max(0, alpha*acc + beta*C) + x_factor*X
};

// ---------------------------------------------------------------------------
// MFMA traits per A/B element type and block size BLK (32: 32x32 output
// blocks, 16: 16x16).  KSB = bytes of K one MFMA consumes per row.  Lane l
// holds row (column) l % BLK of the A (B) block and the (l / BLK)-th equal
// share of those KSB bytes; A and B fragments use the same lane -> k
// assignment, so the contraction is exact whatever order the matrix core
// walks k in.  Accumulator register v of lane l holds output row acc_row(l,
// v) of the block and column l % BLK; registers 4g .. 4g+3 are four
// consecutive rows.
// ---------------------------------------------------------------------------
struct MmaLayout32 {
  static constexpr int BLK = 32, ACCN = 16;
  static __device__ __forceinline__ int acc_row(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
};
struct MmaLayout16 {
  static constexpr int BLK = 16, ACCN = 4;
  static __device__ __forceinline__ int acc_row(int lane, int v) { return 4 * (lane >> 4) + v; }
};

template <int AB, int BLK> struct Mma;

template <> struct Mma<T_F16, 32> : MmaLayout32 {
  typedef v16f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_F16, 16> : MmaLayout16 {
  typedef v4f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_BF16, 32> : MmaLayout32 {
  typedef v16f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_BF16, 16> : MmaLayout16 {
  typedef v4f acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 2, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_I8, 32> : MmaLayout32 {
  typedef v16i acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 1, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<T_I8, 16> : MmaLayout16 {
  typedef v4i acc_t;
  typedef v4i frag_t;
  static constexpr int ESIZE = 1, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};
// Format selectors 0/0 = fp8 e4m3 for both operands; zero scale operands
// select the unscaled instruction.
template <> struct Mma<T_E4M3, 32> : MmaLayout32 {
  typedef v16f acc_t;
  typedef v8i frag_t;
  static constexpr int ESIZE = 1, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
template <> struct Mma<T_E4M3, 16> : MmaLayout16 {
  typedef v4f acc_t;
  typedef v8i frag_t;
  static constexpr int ESIZE = 1, KSB = 128;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

// Format selectors 1/1 = fp8 e5m2 (bf8) for both operands.
template <> struct Mma<T_E5M2, 32> : MmaLayout32 {
  typedef v16f acc_t;
  typedef v8i frag_t;
  static constexpr int ESIZE = 1, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 1, 1, 0, 0, 0, 0);
  }
};

// Mixed fp8 pairs: the f8f6f4 MFMA takes one format selector per operand
// (A first, then B; 0 = e4m3, 1 = e5m2).
template <int FA, int FB>
struct MmaF8Pair : MmaLayout32 {
  typedef v16f acc_t;
  typedef v8i frag_t;
  static constexpr int ESIZE = 1, KSB = 64;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
  }
};
template <> struct Mma<T_E4M3_E5M2, 32> : MmaF8Pair<0, 1> {};
template <> struct Mma<T_E5M2_E4M3, 32> : MmaF8Pair<1, 0> {};

// Eight fp8 values (format F: 0 e4m3, 1 e5m2) widened to fp16.  Every finite
// e4m3 and e5m2 value, subnormals included, is an fp16 value (e4m3: |v| <= 448,
// steps down to 2^-9; e5m2: |v| <= 57344, steps down to 2^-16), so with a scale
// of 1 the conversion is exact, and NaN stays NaN.  Byte i of the input is
// element i of the result.
template <int F>
__device__ __forceinline__ v8h widen8(v2i x) {
  v2h h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned w = (unsigned)(i < 2 ? x.x : x.y);
    if constexpr (F == 0)
      h[i] = (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    else
      h[i] = (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false);
  }
  return v8h{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
}

// fp8 operands (formats FA x FB) in LDS, widened to fp16 in registers for the
// 16x16x32 f16 MFMA: the products and their fp32 sums are those of fp16
// inputs, so fp32 outputs keep fp32's precision (the fp8 MFMA sums a group of
// products with fewer fraction bits).  A k step is 32 bytes of an LDS row;
// lane group q = l / 16 takes bytes [8q, 8q + 8).
template <int FA, int FB>
struct MmaWiden : MmaLayout16 {
  typedef v4f acc_t;
  typedef v2i frag_t;
  static constexpr int ESIZE = 1, KSB = 32;
  static __device__ __forceinline__ acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8<FA>(a), widen8<FB>(b), c, 0, 0, 0);
  }
};
template <> struct Mma<T_W_E4M3, 16> : MmaWiden<0, 0> {};
template <> struct Mma<T_W_E5M2, 16> : MmaWiden<1, 1> {};
template <> struct Mma<T_W_E4M3_E5M2, 16> : MmaWiden<0, 1> {};
template <> struct Mma<T_W_E5M2_E4M3, 16> : MmaWiden<1, 0> {};

// Compile-time kernel configuration.
//   BM x BN     workgroup tile (multiples of 32 per wave)
//   ROWB        K bytes per LDS row per stage (64 or 128)
//   WAVES_M/N   wave grid; each wave owns (BM/WAVES_M) x (BN/WAVES_N)
//   STAGES      depth of the LDS ring
//   DQ          two-stage ring: quarters of a K tile's DMA issued early in
//               step 0 of the K tile before its use (see the mainloop)
//   BLK         MFMA output block: 32 (32x32) or 16 (16x16)
template <int AB_, bool A_KMAJOR_, bool B_KMAJOR_, bool CD_NMAJOR_, int BM_ = 256, int BN_ = 256,
          int ROWB_ = 128, int WAVES_M_ = 2, int WAVES_N_ = 2, int STAGES_ = 2, int DQ_ = 0,
          int BLK_ = 32>
struct Cfg {
  static constexpr int BLK = BLK_;
  using MM = Mma<AB_, BLK_>;
  static constexpr int DQ = DQ_;
  static_assert(DQ >= 0 && DQ <= 4 && (STAGES_ == 2 || DQ == 0), "DQ: quarters, two-stage rings only");
  static constexpr int AB = AB_;
  static constexpr bool A_KMAJOR = A_KMAJOR_, B_KMAJOR = B_KMAJOR_, CD_NMAJOR = CD_NMAJOR_;
  static constexpr int BM = BM_, BN = BN_, ROWB = ROWB_;
  static constexpr int CH = ROWB / 16;                  // 16-byte chunks per LDS row
  static constexpr int ROWS_PER_DMA = 1024 / ROWB;       // rows one wave DMA writes
  static constexpr int SWZ_SHIFT = CH == 8 ? 1 : 2;      // 16 rows -> 16 bank groups
  static constexpr int BK = ROWB / MM::ESIZE;            // K elements per stage
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = NW * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile
  static constexpr int FM = WM / BLK, FN = WN / BLK;         // MFMA output blocks
  // bytes of one k step per lane: lane group q = l / BLK reads bytes
  // [q*BPL, q*BPL + BPL) of the step, i.e. CPL whole 16-byte chunks (or, for
  // BPL = 8, half of chunk q / 2)
  static constexpr int BPL = MM::KSB / (64 / BLK);
  static constexpr int CPL = BPL >= 16 ? BPL / 16 : 1;
  static constexpr int STAGES = STAGES_;
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int PIPE_BYTES = STAGES * STAGE_BYTES;
  // epilogue: per wave, 32 lines of the block being re-laid out
  static constexpr int EPI_LINE = CD_NMAJOR ? WN : WM;
  // words; N-major: the lane groups of one accumulator write (rows 4 apart)
  // land on disjoint banks
  static constexpr int EPI_PITCH = EPI_LINE + (CD_NMAJOR && BLK == 32 ? 8 : 4);
  static constexpr int EPI_WAVE_BYTES = 32 * EPI_PITCH * 4;
  static constexpr int EPI_BYTES = NW * EPI_WAVE_BYTES;
  static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  static constexpr int KSTEPS = ROWB / MM::KSB;
  static_assert(KSTEPS >= 1, "a stage must hold at least one MFMA k step");
  static_assert(BPL * (64 / BLK) == MM::KSB && (BPL == 8 || BPL == 16 || BPL == 32),
                "k step must split evenly over lane groups");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32-line epilogue blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

template <int V>
struct IntC {
  static constexpr int value = V;
  constexpr operator int() const { return V; }
};

// Calls f(IntC<I>{}) for I = B .. E-1, in order, at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Chunk swizzle: the 16-byte chunk c of LDS row r lives at c ^ swz(r).
template <class CF>
__device__ __forceinline__ int swz(int row) {
  return (row >> CF::SWZ_SHIFT) & (CF::CH - 1);
}

// s_waitcnt vmcnt(N) for a compile-time N (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-offs.  Waits only for this wave's LDS
// operations; the DMA stages are covered by the counted vmcnt waits, and
// global stores of the epilogue stay in flight.  (__syncthreads() would add a
// release fence that drains every outstanding memory operation first.)
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Staging of a K-major operand tile (R rows x ROWB bytes) straight into LDS.
// One wave instruction moves 64 chunks = 1 KiB of LDS, written linearly:
// lane j fills physical chunk j % CH of row j / CH, so it fetches the logical
// chunk (j % CH) ^ swz(row) from global memory.
// ---------------------------------------------------------------------------
//
// The DMA is issued through inline asm on purpose: the compiler tracks LDS
// DMA it emits itself and then waits for every outstanding VMEM operation
// before any later LDS read, which would drain the whole ring each K tile.
// Completion is instead tracked here with counted vmcnt waits followed by a
// workgroup barrier.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// The mainloop form: LDS address m0 = sbase + IMM (IMM a compile-time
// constant folded into the m0 write), global offset voff (per lane) + soff
// (the K tile's byte offset, a scalar), so one load costs three issue slots
// and no vector ALU work.
template <uint32_t IMM>
__device__ __forceinline__ void dma16s(v4i rsrc, uint32_t sbase, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_add_u32 m0, %0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(sbase), "v"(voff), "s"(rsrc), "s"(soff), "i"(IMM)
      : "memory", "m0", "scc");
}

// Raw buffer descriptor: base, stride 0, num_records bytes, default format.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = 0x00020000;
  return r;
}

template <class CF, int R>
struct KMajorStager {
  static constexpr int NQ = R / (CF::ROWS_PER_DMA * CF::NW);
  static_assert(NQ * CF::ROWS_PER_DMA * CF::NW == R, "rows must split evenly over the waves");
  // Consecutive instructions of one wave are NW*ROWS_PER_DMA rows apart, a
  // whole number of swizzle periods, so a lane fetches the same logical
  // chunk of its row in every instruction.
  static_assert((CF::NW * CF::ROWS_PER_DMA) % (CF::CH << CF::SWZ_SHIFT) == 0,
                "one chunk offset per lane for all instructions");
  v4i rsrc;
  uint32_t voff[NQ];
  uint32_t cb;  // byte offset of this lane's logical chunk within its row

  __device__ __forceinline__ void setup(const char* tile_base, int64_t ld_bytes, int valid_rows,
                                        int wave, int lane) {
    const int rsub = lane / CF::CH;
    const int pc = lane % CF::CH;
    rsrc = make_rsrc(tile_base, (uint32_t)((int64_t)valid_rows * ld_bytes));
    cb = (uint32_t)((pc ^ swz<CF>(wave * CF::ROWS_PER_DMA + rsub)) * 16);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int row = (q * CF::NW + wave) * CF::ROWS_PER_DMA + rsub;
      voff[q] = (uint32_t)(row * ld_bytes) + cb;
    }
  }

  // Issue instructions [Q0, Q1) of the loads of K tile kt into LDS at byte
  // address lds_addr (LDS address space).  kvalid = bytes of K left from
  // this K tile on; chunks at or past it get an out-of-range offset and read
  // as zero.
  // Instruction Q of a K tile: LDS byte address sbase + REGION + Q*NW KiB
  // (sbase = the stage's address plus this wave's KiB), global offset kofs
  // into each row.  GUARD: kvalid = bytes of K left from kofs (> 0); chunks
  // at or past it read as zero.  Without GUARD the K tile is whole.
  template <int Q, uint32_t REGION, bool GUARD>
  __device__ __forceinline__ void issue_one(uint32_t sbase, uint32_t kofs, int kvalid) {
    uint32_t vo = voff[Q];
    if constexpr (GUARD) vo = (int)cb < kvalid ? vo : 0x80000000u;
    dma16s<REGION + (uint32_t)Q * CF::NW * 1024u>(rsrc, sbase, vo, kofs);
  }

  template <int Q0 = 0, int Q1 = NQ>
  __device__ __forceinline__ void issue(uint32_t lds_addr, int wave, int kt, int64_t kvalid) {
    const uint32_t kofs = (uint32_t)kt * (uint32_t)CF::ROWB;
    if (kvalid >= CF::ROWB) {
#pragma unroll
      for (int q = Q0; q < Q1; ++q)
        dma16(rsrc, lds_addr + (uint32_t)((q * CF::NW + wave) * 1024), voff[q] + kofs);
    } else {
#pragma unroll
      for (int q = Q0; q < Q1; ++q) {
        const uint32_t vo = (int64_t)cb < kvalid ? voff[q] + kofs : 0x80000000u;
        dma16(rsrc, lds_addr + (uint32_t)((q * CF::NW + wave) * 1024), vo);
      }
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
// Staging of an M-major one-byte A tile: global A[l][k][m], ROWB k rows by
// BM m bytes per stage.  Each thread owns blocks of 8 k x 8 m bytes: eight
// 8-byte global loads (a wave covers whole k rows of the tile), an 8x8 byte
// transpose in registers, then eight 8-byte LDS writes into the same
// K-contiguous swizzled layout the K-major path produces.
// ---------------------------------------------------------------------------
template <class CF>
struct MMajorStager8 {
  static constexpr int MB = CF::BM / 8;                       // m blocks per tile
  static constexpr int NB = (CF::ROWB / 8) * MB / CF::THREADS;  // blocks per thread
  static_assert(NB >= 1 && NB * CF::THREADS == (CF::ROWB / 8) * MB, "blocks must split evenly");
  v2u buf[NB][8];
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
      const int id = b * CF::THREADS + tid;
      const int bm = id % MB, bk = id / MB;
      const int64_t m = (int64_t)m0 + bm * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = (int64_t)kt * CF::ROWB + bk * 8 + r;
        if (k < K && m < M)
          buf[b][r] = *(const v2u*)(base + k * M + m);
        else
          buf[b][r] = v2u{0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int lds_off, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = b * CF::THREADS + tid;
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
        const int off = lds_off + row * CF::ROWB + ((chunk ^ swz<CF>(row)) << 4) + sub;
        *(v2u*)(lds + off) = v2u{lo[i], hi[i]};
      }
    }
  }
};

// Fragment read: lane group q's share (BPL bytes) of k step s of LDS row
// row0 + blk*BLK.  Rows BLK apart share their chunk swizzle (a block spans
// whole swizzle periods), so the swizzle is taken from row0 and block blk is
// an immediate offset from block 0's address.
template <class CF>
__device__ __forceinline__ typename CF::MM::frag_t read_frag(const char* lds, int tile_off, int row0, int blk,
                                                             int s, int q) {
  static_assert(CF::BLK % (CF::CH << CF::SWZ_SHIFT) == 0, "block rows span whole swizzle periods");
  const char* rp = lds + tile_off + row0 * CF::ROWB + blk * (CF::BLK * CF::ROWB);
  const int sw = swz<CF>(row0);
  if constexpr (CF::BPL == 8) {
    const int c = s * (CF::MM::KSB / 16) + (q >> 1);
    return *(const v2i*)(rp + ((c ^ sw) << 4) + (q & 1) * 8);
  } else if constexpr (CF::CPL == 1) {
    const int c = s * (CF::MM::KSB / 16) + q;
    return *(const v4i*)(rp + ((c ^ sw) << 4));
  } else {
    const int c = s * (CF::MM::KSB / 16) + q * CF::CPL;
    static_assert(CF::CPL == 2, "one or two chunks per lane");
    const v4i lo = *(const v4i*)(rp + ((c ^ sw) << 4));
    const v4i hi = *(const v4i*)(rp + (((c + 1) ^ sw) << 4));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Accumulator element as the 32-bit pattern stored in LDS.  (The element is
// read into a scalar first: bit-casting a vector-element lvalue directly
// reads element 0 with this compiler.)
__device__ __forceinline__ float acc_bits(float v) { return v; }
__device__ __forceinline__ float acc_bits(int v) { return __int_as_float(v); }

// Writes 32-line block `blk` of this wave's accumulator tile into its LDS
// region (fp32 or int32 bit patterns): for N-major outputs rows blk*32 ..
// blk*32+31 of the wave tile (line = row, WN columns), for M-major columns
// (line = column, WM rows).
template <class CF, class ACC>
__device__ __forceinline__ void epi_stage_block(const ACC (&acc)[CF::FM][CF::FN], float* region, int lane,
                                                int blk) {
  using MM = typename CF::MM;
  constexpr int BLK = CF::BLK, PITCH = CF::EPI_PITCH, SUB = 32 / BLK;
  const int lc = lane % BLK;
  if constexpr (CF::CD_NMAJOR) {
#pragma unroll
    for (int b = 0; b < SUB; ++b)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j)
#pragma unroll
        for (int v = 0; v < MM::ACCN; ++v) {
          const auto x = acc[blk * SUB + b][j][v];
          region[(b * BLK + MM::acc_row(lane, v)) * PITCH + j * BLK + lc] = acc_bits(x);
        }
  } else {
#pragma unroll
    for (int b = 0; b < SUB; ++b)
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int g = 0; g < MM::ACCN / 4; ++g) {
          const auto e0 = acc[i][blk * SUB + b][4 * g + 0], e1 = acc[i][blk * SUB + b][4 * g + 1];
          const auto e2 = acc[i][blk * SUB + b][4 * g + 2], e3 = acc[i][blk * SUB + b][4 * g + 3];
          *(v4f*)(region + (b * BLK + lc) * PITCH + i * BLK + MM::acc_row(lane, 4 * g)) =
              v4f{acc_bits(e0), acc_bits(e1), acc_bits(e2), acc_bits(e3)};
        }
  }
}

// The clamp of the ReLU form: max(0, v), a NaN becoming 0; for int32 the
// signed value of the wrapped sum.
__device__ __forceinline__ v4f relu4(v4f t) {
  return v4f{t.x > 0.0f ? t.x : 0.0f, t.y > 0.0f ? t.y : 0.0f, t.z > 0.0f ? t.z : 0.0f,
             t.w > 0.0f ? t.w : 0.0f};
}
__device__ __forceinline__ v4u relu4(v4u t) {
  return v4u{(int)t.x > 0 ? t.x : 0u, (int)t.y > 0 ? t.y : 0u, (int)t.z > 0 ? t.z : 0u,
             (int)t.w > 0 ? t.w : 0u};
}

// ---------------------------------------------------------------------------
// Epilogue for one element type T shared by every C, X, D and Y in use (the
// common case), same re-layout as above.  Each array is addressed through a
// buffer resource based at this wave's output region with 32-bit offsets:
// rows (N-major) or columns (M-major) past the matrix fall outside the
// resource's extent, so their loads read zero and their stores are dropped
// by the range check; a lane whose 16 bytes lie past the other extent gets
// an offset above 2^31 (the 16-byte rule keeps a lane's group whole).  A skipped term is an empty resource with a zero
// scale; a missing Y is an empty resource.  C and X loads run DIST passes
// ahead of the passes being finished.
// ---------------------------------------------------------------------------
template <int T> struct EpiElem;
template <> struct EpiElem<T_F16> { static constexpr int SIZE = 2; };
template <> struct EpiElem<T_BF16> { static constexpr int SIZE = 2; };
template <> struct EpiElem<T_F32> { static constexpr int SIZE = 4; };
template <> struct EpiElem<T_I32> { static constexpr int SIZE = 4; };

constexpr int EPI_NT = 2;  // cache policy: streaming (non-temporal) access

// One 16-byte access per lane and array: 8 elements of a 2-byte type or 4
// of a 4-byte type.
template <int T>
__device__ __forceinline__ v4u epi_ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, EPI_NT));
}

// Elements [4h, 4h+4) of a 16-byte group as floats.
template <int T>
__device__ __forceinline__ v4f epi_dec(v4u r, int h) {
  const uint32_t a = h ? r.z : r.x, b = h ? r.w : r.y;
  if constexpr (T == T_F16) {
    const v4h f = __builtin_bit_cast(v4h, v2u{a, b});
    return v4f{(float)f.x, (float)f.y, (float)f.z, (float)f.w};
  } else if constexpr (T == T_BF16) {
    return v4f{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u), __uint_as_float(b << 16),
               __uint_as_float(b & 0xffff0000u)};
  } else {
    return __builtin_bit_cast(v4f, r);
  }
}

// Rounds (to nearest even) and packs 4 (4-byte types: lo only) or 8 values.
template <int T>
__device__ __forceinline__ v4u epi_pack(v4f lo, v4f hi) {
  if constexpr (T == T_F16) {
    _Float16 h[8] = {(_Float16)lo.x, (_Float16)lo.y, (_Float16)lo.z, (_Float16)lo.w,
                     (_Float16)hi.x, (_Float16)hi.y, (_Float16)hi.z, (_Float16)hi.w};
    return __builtin_bit_cast(v4u, h);
  } else if constexpr (T == T_BF16) {
    __bf16 b[8] = {(__bf16)lo.x, (__bf16)lo.y, (__bf16)lo.z, (__bf16)lo.w,
                   (__bf16)hi.x, (__bf16)hi.y, (__bf16)hi.z, (__bf16)hi.w};
    return __builtin_bit_cast(v4u, b);
  } else {
    return __builtin_bit_cast(v4u, lo);
  }
}

template <int T>
__device__ __forceinline__ void epi_st(__amdgpu_buffer_rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, EPI_NT);
}

template <class CF, int T, class ACC>
__device__ __forceinline__ void epilogue_typed(const Params& p, const ACC (&acc)[CF::FM][CF::FN], char* lds,
                                               int wave, int lane, int l, int mw, int nw) {
  constexpr bool NMAJ = CF::CD_NMAJOR;
  constexpr int LINE = CF::EPI_LINE, PITCH = CF::EPI_PITCH;
  constexpr int ES = EpiElem<T>::SIZE;
  constexpr int VEC = 16 / ES;         // elements per lane: one 16-byte access per array
  constexpr int LPL = LINE / VEC;      // lanes per line
  constexpr int LINES_PER_PASS = 64 / LPL;
  static_assert(LPL >= 1 && LPL <= 64 && 32 % LINES_PER_PASS == 0, "line split over the lanes");
  float* region = (float*)(lds + wave * CF::EPI_WAVE_BYTES);
  constexpr int NBLK = (NMAJ ? CF::WM : CF::WN) / 32;
  constexpr int PASSES = 32 / LINES_PER_PASS;
  constexpr int NP = NBLK * PASSES;
  constexpr int DIST0 = 8;  // passes of C and X loads in flight: 16 KiB per wave
  constexpr int DIST = DIST0 < NP ? DIST0 : NP;
  const int sub = lane / LPL;
  const int e = (lane % LPL) * VEC;

  // The wave's region: N-major rows [mw, mw+WM) (ld = N), M-major columns
  // [nw, nw+WN) (ld = M); `lines` of them lie inside the matrix.
  const int64_t ld = NMAJ ? p.N : p.M;
  const int64_t line0 = NMAJ ? mw : nw;
  const int64_t nlines = NMAJ ? p.M : p.N;
  const int64_t lines = min(max(nlines - line0, (int64_t)0), (int64_t)(NMAJ ? CF::WM : CF::WN));
  const int64_t slab = ((int64_t)l * (NMAJ ? p.M : p.N) + line0) * ld;  // element index of the base
  const int records = (int)(lines * ld * ES);
  auto rsrc = [&](const void* base, bool live) {
    return __builtin_amdgcn_make_buffer_rsrc(live ? (void*)((const char*)base + slab * ES) : (void*)base,
                                             (short)0, live ? records : 0, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rc = rsrc(p.C ? p.C : p.D, p.C != nullptr);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.X ? p.X : p.D, p.X != nullptr);
  const __amdgpu_buffer_rsrc_t rd = rsrc(p.D, true);
  const __amdgpu_buffer_rsrc_t ry = rsrc(p.Y ? p.Y : p.D, p.Y != nullptr);
  const float beta = p.C ? p.beta : 0.0f;
  const float xf = p.X ? p.xf : 0.0f;
  // along the line: columns (N-major) or rows (M-major) of this lane
  const int64_t along = (NMAJ ? nw : mw) + e;
  const bool lane_ok = along < (NMAJ ? p.N : p.M);
  const uint32_t lane_off = lane_ok ? (uint32_t)((sub * ld + along) * ES) : 0x80000000u;
  auto off = [&](int i) {  // byte offset of pass i (block i / PASSES)
    const int line = (i / PASSES) * 32 + (i % PASSES) * LINES_PER_PASS;
    return lane_off + (uint32_t)(line * ld * ES);
  };

  auto write_block = [&](auto blk_c) { epi_stage_block<CF>(acc, region, lane, decltype(blk_c)::value); };

  v4u cr[DIST + 1], xr[DIST + 1];
  static_for<0, DIST>([&](auto i_c) {
    constexpr int i = decltype(i_c)::value;
    cr[i] = epi_ld<T>(rc, off(i));
    xr[i] = epi_ld<T>(rx, off(i));
  });
  static_for<0, NP>([&](auto i_c) {
    constexpr int i = decltype(i_c)::value, S = i % (DIST + 1);
    constexpr int blk = i / PASSES, ps = i % PASSES;
    // this wave's reads of the previous block are issued before these
    // writes, and LDS serves one wave's operations in order
    if constexpr (ps == 0) write_block(IntC<blk>{});
    const float* wp = region + (ps * LINES_PER_PASS + sub) * PITCH + e;
    const v4f w0 = *(const v4f*)wp;
    const v4f w1 = VEC == 8 ? *(const v4f*)(wp + 4) : v4f{};
    if constexpr (i + DIST < NP) {
      constexpr int SN = (i + DIST) % (DIST + 1);
      cr[SN] = epi_ld<T>(rc, off(i + DIST));
      xr[SN] = epi_ld<T>(rx, off(i + DIST));
    }
    const uint32_t o = off(i);
    if constexpr (T == T_I32) {
      const v4u a = __builtin_bit_cast(v4u, w0);
      v4u t = a * (unsigned)p.ialpha + cr[S] * (unsigned)p.ibeta;
      if (p.relu) t = relu4(t);
      t += xr[S] * (unsigned)p.ix;
      epi_st<T>(rd, o, t);
      epi_st<T>(ry, o, a);
    } else {
      // D = alpha * acc + beta * C (clamped at 0 in the ReLU form) + x_factor * X,
      // in this order
      auto fin = [&](v4f w, int h) {
        const v4f c = epi_dec<T>(cr[S], h), x = epi_dec<T>(xr[S], h);
        v4f t = w * p.alpha;
        t.x = __builtin_fmaf(beta, c.x, t.x);
        t.y = __builtin_fmaf(beta, c.y, t.y);
        t.z = __builtin_fmaf(beta, c.z, t.z);
        t.w = __builtin_fmaf(beta, c.w, t.w);
        if (p.relu) t = relu4(t);
        t.x = __builtin_fmaf(xf, x.x, t.x);
        t.y = __builtin_fmaf(xf, x.y, t.y);
        t.z = __builtin_fmaf(xf, x.z, t.z);
        t.w = __builtin_fmaf(xf, x.w, t.w);
        return t;
      };
      const v4f d0 = fin(w0, 0);
      const v4f d1 = VEC == 8 ? fin(w1, 1) : v4f{};
      epi_st<T>(rd, o, epi_pack<T>(d0, d1));
      epi_st<T>(ry, o, epi_pack<T>(w0, w1));
    }
  });
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Epilogue for C, X, D, Y of different element types (f16, bf16, f32): the
// same re-layout, addressing and load-ahead as the one-type epilogue, with 4
// elements per lane (16 bytes of a 4-byte type, 8 of a 2-byte type) and each
// array's element size, decoding and rounding chosen by its (uniform) type,
// so no lane takes a branch of its own.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4u epi_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off, bool wide) {
  if (wide) return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, EPI_NT));
  const v2u u = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, EPI_NT));
  return v4u{u.x, u.y, 0u, 0u};
}

// Raw bits of four elements of type dt -> four fp32 values.
__device__ __forceinline__ v4f epi_decode4(v4u r, int dt) {
  if (dt == T_F32) return __builtin_bit_cast(v4f, r);
  if (dt == T_BF16)
    return v4f{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
               __uint_as_float(r.y & 0xffff0000u)};
  const v4h h = __builtin_bit_cast(v4h, v2u{r.x, r.y});
  return v4f{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
}

// Rounds four fp32 values to nearest-even into type dt and stores them.
__device__ __forceinline__ void epi_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, int dt, v4f v) {
  if (dt == T_F16) {
    const v4h h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, h), r, (int)off, 0, EPI_NT);
  } else if (dt == T_BF16) {
    const v4bf b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, b), r, (int)off, 0, EPI_NT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)off, 0, EPI_NT);
  }
}

__device__ __forceinline__ int epi_shift(int dt) { return dt == T_F32 || dt == T_I32 ? 2 : 1; }

template <class CF, class ACC>
__device__ __forceinline__ void epilogue_mixed(const Params& p, const ACC (&acc)[CF::FM][CF::FN], char* lds,
                                               int wave, int lane, int l, int mw, int nw) {
  constexpr bool NMAJ = CF::CD_NMAJOR;
  constexpr int LINE = CF::EPI_LINE, PITCH = CF::EPI_PITCH;
  constexpr int VEC = 4;
  constexpr int LPL = LINE / VEC;
  constexpr int LINES_PER_PASS = 64 / LPL;
  static_assert(LPL >= 1 && LPL <= 64 && 32 % LINES_PER_PASS == 0, "line split over the lanes");
  float* region = (float*)(lds + wave * CF::EPI_WAVE_BYTES);
  constexpr int NBLK = (NMAJ ? CF::WM : CF::WN) / 32;
  constexpr int PASSES = 32 / LINES_PER_PASS;
  constexpr int NP = NBLK * PASSES;
  constexpr int DIST0 = 8;
  constexpr int DIST = DIST0 < NP ? DIST0 : NP;
  const int sub = lane / LPL;
  const int e = (lane % LPL) * VEC;

  const int64_t ld = NMAJ ? p.N : p.M;
  const int64_t line0 = NMAJ ? mw : nw;
  const int64_t nlines = NMAJ ? p.M : p.N;
  const int64_t lines = min(max(nlines - line0, (int64_t)0), (int64_t)(NMAJ ? CF::WM : CF::WN));
  const int64_t slab = ((int64_t)l * (NMAJ ? p.M : p.N) + line0) * ld;  // element index of the base
  auto rsrc = [&](const void* base, int dt) {
    const int sh = epi_shift(dt);
    return __builtin_amdgcn_make_buffer_rsrc(base ? (void*)((const char*)base + (slab << sh)) : (void*)p.D,
                                             (short)0, base ? (int)((lines * ld) << sh) : 0, 0x00020000);
  };
  const int tc = p.C ? p.c_dtype : T_F32, tx = p.X ? p.x_dtype : T_F32, td = p.d_dtype;
  const int ty = p.Y ? p.y_dtype : T_F32;
  const __amdgpu_buffer_rsrc_t rc = rsrc(p.C, tc), rx = rsrc(p.X, tx), rd = rsrc(p.D, td), ry = rsrc(p.Y, ty);
  const int shc = epi_shift(tc), shx = epi_shift(tx), shd = epi_shift(td), shy = epi_shift(ty);
  const float beta = p.C ? p.beta : 0.0f;
  const float xf = p.X ? p.xf : 0.0f;
  const int64_t along = (NMAJ ? nw : mw) + e;
  const bool lane_ok = along < (NMAJ ? p.N : p.M);
  // element offset of this lane in pass i; a lane past the other extent gets
  // a byte offset above 2^31 in every array (outside every resource)
  const uint32_t lane_el = (uint32_t)(sub * ld + along);
  auto el = [&](int i) {
    const int line = (i / PASSES) * 32 + (i % PASSES) * LINES_PER_PASS;
    return lane_el + (uint32_t)(line * ld);
  };
  auto boff = [&](uint32_t eo, int sh) { return lane_ok ? eo << sh : 0x80000000u; };

  auto write_block = [&](auto blk_c) { epi_stage_block<CF>(acc, region, lane, decltype(blk_c)::value); };

  v4u cr[DIST + 1], xr[DIST + 1];
  static_for<0, DIST>([&](auto i_c) {
    constexpr int i = decltype(i_c)::value;
    cr[i] = epi_ld4(rc, boff(el(i), shc), shc == 2);
    xr[i] = epi_ld4(rx, boff(el(i), shx), shx == 2);
  });
  static_for<0, NP>([&](auto i_c) {
    constexpr int i = decltype(i_c)::value, S = i % (DIST + 1);
    constexpr int blk = i / PASSES, ps = i % PASSES;
    if constexpr (ps == 0) write_block(IntC<blk>{});
    const v4f w = *(const v4f*)(region + (ps * LINES_PER_PASS + sub) * PITCH + e);
    if constexpr (i + DIST < NP) {
      constexpr int SN = (i + DIST) % (DIST + 1);
      cr[SN] = epi_ld4(rc, boff(el(i + DIST), shc), shc == 2);
      xr[SN] = epi_ld4(rx, boff(el(i + DIST), shx), shx == 2);
    }
    const uint32_t eo = el(i);
    // D = alpha * acc + beta * C (clamped at 0 in the ReLU form) + x_factor * X
    const v4f c = epi_decode4(cr[S], tc), x = epi_decode4(xr[S], tx);
    v4f t = w * p.alpha;
    t.x = __builtin_fmaf(beta, c.x, t.x);
    t.y = __builtin_fmaf(beta, c.y, t.y);
    t.z = __builtin_fmaf(beta, c.z, t.z);
    t.w = __builtin_fmaf(beta, c.w, t.w);
    if (p.relu) t = relu4(t);
    t.x = __builtin_fmaf(xf, x.x, t.x);
    t.y = __builtin_fmaf(xf, x.y, t.y);
    t.z = __builtin_fmaf(xf, x.z, t.z);
    t.w = __builtin_fmaf(xf, x.w, t.w);
    epi_st4(rd, boff(eo, shd), td, t);
    if (p.Y) epi_st4(ry, boff(eo, shy), ty, w);
  });
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Scheduling pattern for one k step: READS LDS reads spread evenly over
// MFMAS matrix instructions ([1 read, MFMAS/READS MFMAs] repeated).
template <int R, int READS, int MFMAS>
struct InterleaveHint {
  static __device__ __forceinline__ void run() {
    if constexpr (R < READS) {
      constexpr int n = MFMAS / READS + (R < MFMAS % READS ? 1 : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x008, n, 0);  // MFMAs
      InterleaveHint<R + 1, READS, MFMAS>::run();
    }
  }
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <class CF>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_epi_kernel(Params p) {
  using MM = typename CF::MM;
  using acc_t = typename MM::acc_t;
  using frag_t = typename MM::frag_t;
  constexpr int ES = MM::ESIZE;
  constexpr int BM = CF::BM, BN = CF::BN, S = CF::STAGES;
  __shared__ __attribute__((aligned(1024))) char lds[CF::LDS_BYTES];
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)(lds_void_t*)lds;  // LDS address of the array

  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % CF::WAVES_M, wn = wave / CF::WAVES_M;
  const int lq = lane / CF::BLK, lr = lane % CF::BLK;  // k share and row of this lane in a block


  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int g = p.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  const int64_t kbytes = p.K * ES;
  const int KT = (int)((kbytes + CF::ROWB - 1) / CF::ROWB);
  const int64_t tiles_mn = (int64_t)p.tiles_m * p.tiles_n;

  // DMA instructions per wave per stage (for the counted waits)
  constexpr int NQ_A = CF::A_KMAJOR ? KMajorStager<CF, BM>::NQ : 0;
  constexpr int NQ_STAGE = NQ_A + KMajorStager<CF, BN>::NQ;

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
    KMajorStager<CF, BN> sb;
    sb.setup(Bb + (int64_t)n0 * kbytes, kbytes, (int)min((int64_t)BN, p.N - n0), wave, lane);
    KMajorStager<CF, BM> sa_k;
    if constexpr (CF::A_KMAJOR)
      sa_k.setup(Ab + (int64_t)m0 * kbytes, kbytes, (int)min((int64_t)BM, p.M - m0), wave, lane);

    auto issue_dma = [&](int k_tile) {
      const int st = (k_tile % S) * CF::STAGE_BYTES;
      const int64_t kv = kbytes - (int64_t)k_tile * CF::ROWB;
      if constexpr (CF::A_KMAJOR) sa_k.issue(lds_u32 + st, wave, k_tile, kv);
      sb.issue(lds_u32 + st + BM * CF::ROWB, wave, k_tile, kv);
    };
    // Part PART of NPARTS of the loads of K tile k_tile (A and B split alike).
    using SA = KMajorStager<CF, BM>;
    using SB = KMajorStager<CF, BN>;
    auto issue_dma_part = [&](auto part_c, auto nparts_c, int k_tile) {
      constexpr int PART = decltype(part_c)::value, NP = decltype(nparts_c)::value;
      const int st = (k_tile % S) * CF::STAGE_BYTES;
      const int64_t kv = kbytes - (int64_t)k_tile * CF::ROWB;
      if constexpr (CF::A_KMAJOR)
        sa_k.template issue<PART * SA::NQ / NP, (PART + 1) * SA::NQ / NP>(lds_u32 + st, wave, k_tile, kv);
      sb.template issue<PART * SB::NQ / NP, (PART + 1) * SB::NQ / NP>(lds_u32 + st + BM * CF::ROWB, wave,
                                                                      k_tile, kv);
    };

    acc_t acc[CF::FM][CF::FN];
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) acc[i][j] = acc_t{};

    // Fragments of one k step: A blocks then B blocks of this wave.
    frag_t fa[2][CF::FM], fb[2][CF::FN];
    auto load_step = [&](frag_t (&ra)[CF::FM], frag_t (&rb)[CF::FN], int st, int s) {
      const int a_off = st * CF::STAGE_BYTES, b_off = a_off + BM * CF::ROWB;
#pragma unroll
      for (int i = 0; i < CF::FM; ++i) ra[i] = read_frag<CF>(lds, a_off, wm * CF::WM + lr, i, s, lq);
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) rb[j] = read_frag<CF>(lds, b_off, wn * CF::WN + lr, j, s, lq);
    };
    auto mma_step = [&](const frag_t (&ra)[CF::FM], const frag_t (&rb)[CF::FN]) {
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int j = 0; j < CF::FN; ++j) acc[i][j] = MM::mma(ra[i], rb[j], acc[i][j]);
    };
    // Interleave the next step's LDS reads with this step's MFMAs so each
    // read's latency hides under MFMAs already queued.
    auto pipeline_hint = [&]() {
      constexpr int READS = (CF::FM + CF::FN) * CF::CPL;
      constexpr int MFMAS = CF::FM * CF::FN;
      InterleaveHint<0, READS, MFMAS>::run();
    };
    // One K tile from stage st; the last step prefetches step 0 of stage nst.
    // The DMA of K tile dma_tile (if < KT) is issued in NP parts after the
    // first NP k steps, so the memory pipeline is fed while MFMAs run rather
    // than in one burst that stalls the wave's issue.
    auto compute = [&](int st, int nst, int dma_tile, auto np_c) {
      constexpr int NP = decltype(np_c)::value;
      static_for<0, CF::KSTEPS>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int cur = s & 1;
        if constexpr (s + 1 < CF::KSTEPS)
          load_step(fa[cur ^ 1], fb[cur ^ 1], st, s + 1);
        else
          load_step(fa[cur ^ 1], fb[cur ^ 1], nst, 0);
        mma_step(fa[cur], fb[cur]);
        pipeline_hint();
        if constexpr (s < NP) {
          if (dma_tile < KT) issue_dma_part(IntC<s>{}, IntC<NP>{}, dma_tile);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    static_assert(CF::KSTEPS % 2 == 0, "fragment double buffer needs an even step count");

    // ---- K-major A: explicitly ordered k steps ---------------------------
    // Each k step issues its MFMAs in a fixed order (sched_barrier pins it);
    // after each MFMA come the fragment reads of the next step scheduled
    // there (ordered by first use: A0, B0.., A1..) and a share of the DMA
    // instructions of a later K tile, so LDS reads, DMA and MFMAs overlap.
    constexpr int NREAD = CF::FM + CF::FN;
    constexpr int MF = CF::FM * CF::FN;
    auto read_r = [&](auto buf_c, auto r_c, auto st_x, auto ks_x) {
      constexpr int BUF = decltype(buf_c)::value, R = decltype(r_c)::value;
      const int st = (int)st_x, ks = (int)ks_x;
      const int a_off = st * CF::STAGE_BYTES, b_off = a_off + BM * CF::ROWB;
      if constexpr (R == 0)
        fa[BUF][0] = read_frag<CF>(lds, a_off, wm * CF::WM + lr, 0, ks, lq);
      else if constexpr (R <= CF::FN)
        fb[BUF][R - 1] = read_frag<CF>(lds, b_off, wn * CF::WN + lr, R - 1, ks, lq);
      else
        fa[BUF][R - CF::FN] = read_frag<CF>(lds, a_off, wm * CF::WM + lr, R - CF::FN, ks, lq);
    };
    // DMA instruction D of K tile k_tile into stage stg.  GUARD: the tile
    // may not exist (k_tile >= KT) or may be cut by the end of K; without
    // it the tile is whole and no check is made.
    const uint32_t lds_wave = lds_u32 + (uint32_t)wave * 1024u;
    auto dma_one = [&](auto d_c, auto guard_c, int k_tile, int stg) {
      constexpr int D = decltype(d_c)::value;
      constexpr bool GUARD = decltype(guard_c)::value;
      if (GUARD && k_tile >= KT) return;
      const uint32_t sbase = lds_wave + (uint32_t)stg * (uint32_t)CF::STAGE_BYTES;
      const uint32_t kofs = (uint32_t)k_tile * (uint32_t)CF::ROWB;
      const int kv = GUARD ? (int)min(kbytes - (int64_t)kofs, (int64_t)CF::ROWB) : CF::ROWB;
      if constexpr (D < NQ_A)
        sa_k.template issue_one<D, 0u, GUARD>(sbase, kofs, kv);
      else
        sb.template issue_one<D - NQ_A, (uint32_t)(BM * CF::ROWB), GUARD>(sbase, kofs, kv);
    };
    // One k step on buffer CUR: reads of (stage rst, step rs) into CUR^1 and
    // NOPS memory operations op(IntC<k>) spread evenly over the MFMAs.
    auto kstep_ops = [&](auto cur_c, auto rst, auto rs, auto nops_c, auto&& op, auto win_c) {
      constexpr int CUR = decltype(cur_c)::value;
      constexpr int NOPS = decltype(nops_c)::value;
      constexpr int WIN = decltype(win_c)::value;  // ops go among the first WIN MFMAs
      static_for<0, MF>([&](auto idx_c) {
        constexpr int IDX = decltype(idx_c)::value;
        constexpr int I = IDX / CF::FN, J = IDX % CF::FN;
        acc[I][J] = MM::mma(fa[CUR][I], fb[CUR][J], acc[I][J]);
        static_for<0, NREAD>([&](auto r_c) {
          constexpr int R = decltype(r_c)::value;
          if constexpr ((R * MF) / NREAD == IDX) read_r(IntC<CUR ^ 1>{}, r_c, rst, rs);
        });
        if constexpr (NOPS > 0) {
          static_for<0, NOPS>([&](auto k_c) {
            constexpr int KK = decltype(k_c)::value;
            if constexpr (((2 * KK + 1) * WIN) / (2 * NOPS) == IDX) op(k_c);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // DMA variant: instructions [D0, D1) of K tile dma_tile into stage dst,
    // spread over the first WIN MFMAs of the step.
    auto kstep = [&](auto cur_c, auto rst, auto rs, auto d0_c, auto d1_c, auto guard_c, int dma_tile,
                     int dst, auto win_c) {
      constexpr int D0 = decltype(d0_c)::value, D1 = decltype(d1_c)::value;
      kstep_ops(cur_c, rst, rs, IntC<D1 - D0>{}, [&](auto k_c) {
        dma_one(IntC<D0 + decltype(k_c)::value>{}, guard_c, dma_tile, dst);
      }, win_c);
    };
    // Wait until at most `pend` DMA groups (K tiles) of this wave are in
    // flight (loads complete in order).
    auto wait_pending = [&](int pend) {
      if constexpr (S >= 4) {
        if (pend >= 3) wait_vmcnt<3 * NQ_STAGE>();
        else if (pend == 2) wait_vmcnt<2 * NQ_STAGE>();
        else if (pend == 1) wait_vmcnt<NQ_STAGE>();
        else wait_vmcnt<0>();
      } else if constexpr (S == 3) {
        if (pend >= 1) wait_vmcnt<NQ_STAGE>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
    };
    // Where the DMA of one K tile goes.  Deep ring (S >= 3): KSTEPS equal
    // parts, part 0 in the last step of K tile kt-S (right after the barrier
    // that frees its stage) and part q in step q-1 of K tile kt-S+1, so the
    // texture path (64 B/clk per CU, about half of what the MFMAs consume at
    // full rate) is fed evenly and a tile lands S-2 K tiles before it is
    // read.  Two stages: the instructions [0, P0) go over the last step of K
    // tile kt-2 and the remaining DQ quarters [P0, NQ) over the first half
    // of step 0 of K tile kt-1, so that even the last of them lands with
    // half a step to spare before the wait that precedes the last step.
    constexpr int NPARTS = S == 2 ? 1 : CF::KSTEPS;
    constexpr int P0 = S == 2 ? NQ_STAGE - NQ_STAGE * CF::DQ / 4 : NQ_STAGE / NPARTS;
    static_assert(S != 2 || CF::KSTEPS >= 2 || CF::DQ == 0, "an early part needs a step before the last");
    // K tile kt from stage st; nst = stage of kt+1, pst = stage of kt-1
    // (which tile t1 = kt+S-1 refills).  GUARD: DMA checks are needed.
    auto k_tile = [&](auto guard_c, int kt, auto st, auto nst, auto pst, int t1) {
      constexpr bool GUARD = decltype(guard_c)::value;
      static_for<0, CF::KSTEPS - 1>([&](auto s_c) {
        constexpr int SS = decltype(s_c)::value;
        if constexpr (S == 2 && SS == 0 && P0 < NQ_STAGE)
          kstep(IntC<0>{}, st, IntC<1>{}, IntC<P0>{}, IntC<NQ_STAGE>{}, guard_c, t1, (int)pst, IntC<MF / 2>{});
        else if constexpr (S != 2)
          kstep(IntC<SS & 1>{}, st, IntC<SS + 1>{}, IntC<(SS + 1) * NQ_STAGE / NPARTS>{},
                IntC<(SS + 2) * NQ_STAGE / NPARTS>{}, guard_c, t1, (int)pst, IntC<MF>{});
        else
          kstep(IntC<SS & 1>{}, st, IntC<SS + 1>{}, IntC<0>{}, IntC<0>{}, guard_c, t1, (int)pst, IntC<MF>{});
      });
      // Tile kt+1 (read by the last step) must be complete; the groups
      // issued after it (deep ring: min(S-2, KT-2-kt) whole tiles) may pend.
      if constexpr (S == 2) wait_vmcnt<0>();
      else if constexpr (GUARD) wait_pending(min(S - 2, KT - 2 - kt));
      else wait_vmcnt<(S - 2) * NQ_STAGE>();
      barrier_lds();  // tile kt+1 visible; every wave is done reading stage kt
      // Last step: its fragments are in registers; read step 0 of tile kt+1
      // meanwhile and refill stage kt (free now) with part 0 of tile kt+S.
      kstep(IntC<(CF::KSTEPS - 1) & 1>{}, nst, IntC<0>{}, IntC<0>{}, IntC<P0>{}, guard_c, kt + S, (int)st,
            IntC<MF>{});
    };

    if constexpr (CF::A_KMAJOR) {
      static_assert(CF::KSTEPS % 2 == 0, "k steps alternate fragment buffers across K tiles");
      // Prologue: two stages: K tiles 0 and 1 whole, tile 0 complete.  Deep
      // ring: K tiles 0 .. S-2 whole, tile 0 complete, then part 0 of tile
      // S-1 (stage S-1 is untouched so far).
      if constexpr (S == 2) {
        issue_dma(0);
        if (1 < KT) {
          issue_dma(1);
          wait_vmcnt<NQ_STAGE>();
        } else {
          wait_vmcnt<0>();
        }
      } else {
#pragma unroll
        for (int k = 0; k < S - 1; ++k)
          if (k < KT) issue_dma(k);
        wait_pending(min(S - 1, KT) - 1);
        // (tile numbers known at compile time are hidden from constant
        // folding: the DMA's scalar offset operand takes no literal)
        int t_pro = S - 1;
        asm("" : "+s"(t_pro));
        static_for<0, P0>([&](auto d_c) { dma_one(d_c, IntC<1>{}, t_pro, S - 1); });
      }
      barrier_lds();
      load_step(fa[0], fb[0], 0, 0);
      // Guarded K tiles: the first one of the two-stage ring (its tile 1 was
      // issued whole) and every K tile whose loads reach past the last whole
      // K tile; the rest run without checks.
      const int kt_whole = (int)(kbytes / CF::ROWB);
      int kt = 0, st = 0;
      auto next = [](int x) { return x + 1 == S ? 0 : x + 1; };
      auto prev = [](int x) { return x == 0 ? S - 1 : x - 1; };
      if constexpr (S == 2) {
        k_tile(IntC<1>{}, 0, 0, 1, 1, KT);
        kt = 1;
        st = 1;
      }
      if constexpr (S == 2) {
        // Two stages: K tiles in pairs with the stage a compile-time
        // constant, so every fragment address is a loop-invariant register
        // plus an immediate (no address arithmetic between the MFMAs).
        if (kt + S < kt_whole && st == 1) {
          k_tile(IntC<0>{}, kt, IntC<1>{}, IntC<0>{}, IntC<0>{}, kt + S - 1);
          ++kt;
          st = 0;
        }
        for (; kt + 1 + S < kt_whole; kt += 2) {
          k_tile(IntC<0>{}, kt, IntC<0>{}, IntC<1>{}, IntC<1>{}, kt + S - 1);
          k_tile(IntC<0>{}, kt + 1, IntC<1>{}, IntC<0>{}, IntC<0>{}, kt + S);
        }
      }
      for (; kt + S < kt_whole; ++kt) {
        k_tile(IntC<0>{}, kt, st, next(st), prev(st), kt + S - 1);
        st = next(st);
      }
      for (; kt < KT; ++kt) {
        k_tile(IntC<1>{}, kt, st, next(st), prev(st), kt + S - 1);
        st = next(st);
      }
      wait_vmcnt<0>();
    } else {
      // ---- M-major one-byte A: registers + transpose, B by DMA -----------
      MMajorStager8<CF> sa_m;
      sa_m.setup(Ab, p.M, p.K, m0);
      sa_m.load(0, tid);
      sa_m.store(lds, 0, tid);
      sb.issue(lds_u32 + BM * CF::ROWB, wave, 0, kbytes);
      for (int kt = 0; kt < KT; ++kt) {
        wait_vmcnt<0>();
        barrier_lds();  // stage kt complete; stage kt+1 free
        const bool more = kt + 1 < KT;
        const int nxt = ((kt + 1) % S) * CF::STAGE_BYTES;
        if (more) {
          sa_m.load(kt + 1, tid);
          sb.issue(lds_u32 + nxt + BM * CF::ROWB, wave, kt + 1, kbytes - (int64_t)(kt + 1) * CF::ROWB);
        }
        load_step(fa[0], fb[0], kt % S, 0);
        compute(kt % S, kt % S, KT, IntC<0>{});
        if (more) sa_m.store(lds, nxt, tid);
      }
    }
    barrier_lds();  // every wave is done reading the ring

    // ---- fused epilogue ---------------------------------------------------
    const int emw = m0 + wm * CF::WM, enw = n0 + wn * CF::WN;
    if constexpr (CF::AB == T_I8) {
      epilogue_typed<CF, T_I32>(p, acc, lds, wave, lane, l, emw, enw);
    } else {
      if (p.epi_kind == T_F16) epilogue_typed<CF, T_F16>(p, acc, lds, wave, lane, l, emw, enw);
      else if (p.epi_kind == T_BF16) epilogue_typed<CF, T_BF16>(p, acc, lds, wave, lane, l, emw, enw);
      else if (p.epi_kind == T_F32) epilogue_typed<CF, T_F32>(p, acc, lds, wave, lane, l, emw, enw);
      else epilogue_mixed<CF>(p, acc, lds, wave, lane, l, emw, enw);
    }
    barrier_lds();  // LDS is reused by the next tile's prologue
  }
}

}  // namespace gemm_epi
