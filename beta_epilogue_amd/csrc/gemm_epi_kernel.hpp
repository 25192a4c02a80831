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
//   * global -> LDS staging into a STAGES-deep ring by buffer_load_dwordx4
//     ... lds (the buffer's range check turns rows past M/N and chunks past K
//     into zeros).  K-major operands: each LDS row holds ROWB bytes of K of
//     one tile row as 16-byte chunks stored at chunk ^ swz(row), so the
//     MFMA fragment reads of 16 consecutive rows hit 16 distinct 16-byte
//     bank groups of the 64-bank LDS.  M-major A / N-major B: swizzled
//     k-rows, read back with the transposing ds_read_b64_tr_b16/_tr_b8.
//     Each K tile waits only for its own stage (counted vmcnt), so STAGES-1
//     tiles stay in flight (the multi-stage pipeline of the API card's
//     "Depth and shared memory");
//   * MFMA mainloop on 16x16 or 32x32 accumulator blocks in AGPRs:
//     v_mfma_f32_{16x16x32,32x32x16}_{f16,bf16},
//     v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4 (per-operand fp8 format
//     selectors, scales fixed at 1) or v_mfma_i32_{16x16x64,32x32x32}_i8;
//     the fragments of k step s+1 are read while step s multiplies;
//   * fused epilogue on the fp32 (int32) accumulator: Y = acc, D = alpha*acc
//     + beta*C + x_factor*X, rounded to nearest-even into the output types;
//     each 32-wide block of the accumulator is re-laid out through a small
//     per-wave LDS region so C/X loads and D/Y stores move 16 contiguous
//     bytes per lane; all loads of an element precede its stores (the
//     example's epilogue comment) and C and X are only read;
//   * split K: a work item is a whole tile, or one K slice of a tile whose
//     fp32 (int32) partial sums go to a workspace slot; a second kernel adds
//     the slices and applies the epilogue (gemm_epi_splitk.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_epi_raster.hpp"

namespace gemm_epi {

// Element type codes; the same numbers as the public header.
enum : int { T_NONE = 0, T_F16 = 1, T_BF16 = 2, T_E4M3 = 3, T_I8 = 4, T_F32 = 5, T_I32 = 6, T_E5M2 = 7 };
// Kernel A/B codes of the fp8 pairs (A's format x B's).
enum : int { T_E4M3_E5M2 = 8, T_E5M2_E4M3 = 9 };
// Kernel A/B code of uint8: the int8 MFMA on copies of A and B with every
// byte's top bit flipped, the accumulators started at the sums' correction.
enum : int { T_U8 = 14 };

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
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
  int32_t tiles_total;  // work items (below 2^31)
  int32_t L, tiles_m, tiles_n, group_m;
  int32_t c_dtype, x_dtype, d_dtype, y_dtype;  // T_NONE for skipped terms
  float alpha, beta, xf;
  int32_t ialpha, ibeta, ix;  // integral scalars for int32 outputs
  int32_t xcd_remap;          // grid is a multiple of 8: remap ids per XCD
  int32_t epi_kind;           // element type shared by every C/X/D/Y in use (0: mixed)
  int32_t relu;               // D = max(0, alpha*acc + beta*C) + x_factor*X
  // Split K.  Work items 0 .. dp_tiles-1 are the first dp_tiles tiles of
  // the raster, each over the whole K range with the epilogue.  The other
  // tail_tiles tiles are cut into `splits` K slices of kslice elements (a
  // multiple of the K tile; the last one may be shorter): item dp_tiles +
  // s*tail_tiles + j is slice s of tile dp_tiles + j, and it writes its fp32
  // (int32) partial sums, unscaled, to workspace slot s*tail_tiles + j
  // (tile_m*tile_n*4 bytes at ws + slot*tile_m*tile_n*4, holding the tile's
  // rows x cols inside the matrix packed in D's majorness) instead of running
  // the epilogue; a second kernel adds the slices and applies the epilogue.
  // No split: dp_tiles == all tiles, tail_tiles == 0, ws unused.
  int32_t dp_tiles, tail_tiles;
  int32_t splits;
  int64_t kslice;
  void* ws;
  // uint8 A/B on the int8 kernels: A and B here are copies of the unsigned
  // operands with every byte's top bit flipped (u - 128 as a signed byte),
  // so the MFMA sums (u_a - 128)(u_b - 128); each tile's accumulator starts
  // at 128*(rsum_a[m] + rsum_b[n]) + u8_bias with u8_bias = -16384*K
  // (wrapping), which makes it sum u_a*u_b (k past K reads zero and adds
  // nothing).  rsum_a (L x M) and rsum_b (L x N) hold the sums along K of the
  // unsigned bytes.  NULL for int8.
  const int32_t* rsum_a;
  const int32_t* rsum_b;
  int32_t u8_bias;
  // int32 outputs whose scalars need no multiply: ialpha == 1 and ibeta (ix)
  // is 1 or its term skipped (an empty resource reads zero), so
  // D = acc + C + X with adds only (v_mul_lo_u32 is a quarter-rate
  // instruction, three per output otherwise).
  int32_t int_unit;
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

template <> struct Mma<T_U8, 16> : Mma<T_I8, 16> {};
template <> struct Mma<T_U8, 32> : Mma<T_I8, 32> {};

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
  static constexpr bool INT = AB_ == T_I8 || AB_ == T_U8;  // int32 accumulators and epilogue
  static constexpr bool U8 = AB_ == T_U8;
  using RAW = typename MM::frag_t;  // a fragment as read from LDS
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
  // [q*BPL, q*BPL + BPL) of the step, i.e. CPL whole 16-byte chunks
  static constexpr int BPL = MM::KSB / (64 / BLK);
  static constexpr int CPL = BPL / 16;
  static constexpr int STAGES = STAGES_;
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int PIPE_BYTES = STAGES * STAGE_BYTES;
  // epilogue: per wave, 32 lines of the block being re-laid out; lines are
  // rows (N-major C/D: WN floats each) or columns (M-major: WM floats)
  static constexpr int epi_line(bool nmaj) { return nmaj ? WN : WM; }
  // words; N-major: the lane groups of one accumulator write (rows 4 apart)
  // land on disjoint banks
  static constexpr int epi_pitch(bool nmaj) { return epi_line(nmaj) + (nmaj && BLK == 32 ? 8 : 4); }
  static constexpr int epi_wave_bytes(bool nmaj) { return 32 * epi_pitch(nmaj) * 4; }
  static constexpr int EPI_BYTES = NW * epi_wave_bytes(CD_NMAJOR);
  static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  static constexpr int KSTEPS = ROWB / MM::KSB;
  static_assert(KSTEPS >= 1, "a stage must hold at least one MFMA k step");
  static_assert(BPL * (64 / BLK) == MM::KSB && (BPL == 16 || BPL == 32),
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
// Operand tiles in LDS.  Each operand (A: BM rows, B: BN rows) owns a region
// of STAGES stages; a stage holds one K tile of BK elements.  The DMA that
// fills a stage is issued through inline asm on purpose: the compiler tracks
// LDS DMA it emits itself and then waits for every outstanding VMEM
// operation before any later LDS read, which would drain the whole ring
// each K tile.  Completion is tracked with counted vmcnt waits followed by a
// workgroup barrier.  One wave instruction moves 64 chunks of 16 bytes = 1
// KiB, written to LDS linearly; the swizzle of a layout is applied on the
// global side (lane j fetches whichever chunk belongs in LDS chunk j).
// ---------------------------------------------------------------------------
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

typedef __attribute__((address_space(3))) char lds_char_t;
typedef short v4s __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// K-major operand (A 'K' or B 'K'): R rows x ROWB bytes of K per stage; the
// 16-byte chunk c of row r is stored at c ^ swz(r).  Rows past the matrix
// read as zero through the buffer's range check (its extent ends with the
// tile's last row), chunks past K through an out-of-range offset.
// ---------------------------------------------------------------------------
template <class CF, int R, int WR>
struct KMajorOperand {
  static constexpr int NQ = R / (CF::ROWS_PER_DMA * CF::NW);
  static_assert(NQ * CF::ROWS_PER_DMA * CF::NW == R, "rows must split evenly over the waves");
  // Consecutive instructions of one wave are NW*ROWS_PER_DMA rows apart, a
  // whole number of swizzle periods, so a lane fetches the same logical
  // chunk of its row in every instruction.
  static_assert((CF::NW * CF::ROWS_PER_DMA) % (CF::CH << CF::SWZ_SHIFT) == 0,
                "one chunk offset per lane for all instructions");
  v4i rsrc;
  uint32_t voff;   // global byte offset of this lane's chunk in instruction 0
  uint32_t qstep;  // bytes between consecutive instructions (NW * ROWS_PER_DMA rows)
  uint32_t cb;     // byte offset of this lane's logical chunk within its row
  int row0, q;     // reader: LDS row of this lane in block 0, its k share

  // batch: the operand's batch l; extent: M (A) or N (B); K: the full K
  // (the row length); kbeg: the first k of the K range staged (a K slice);
  // r0: the tile's first row.
  __device__ __forceinline__ void setup(const char* batch, int64_t extent, int64_t K, int64_t kbeg, int r0,
                                        int wave, int lane) {
    const int64_t ld_bytes = K * CF::MM::ESIZE;
    const int64_t kb = kbeg * CF::MM::ESIZE;
    const int rsub = lane / CF::CH;
    const int pc = lane % CF::CH;
    const int valid_rows = (int)min((int64_t)R, extent - r0);
    rsrc = make_rsrc(batch + (int64_t)r0 * ld_bytes + kb, (uint32_t)((int64_t)valid_rows * ld_bytes - kb));
    cb = (uint32_t)((pc ^ swz<CF>(wave * CF::ROWS_PER_DMA + rsub)) * 16);
    voff = (uint32_t)((wave * CF::ROWS_PER_DMA + rsub) * ld_bytes) + cb;
    qstep = (uint32_t)(CF::NW * CF::ROWS_PER_DMA * ld_bytes);
  }
  // rbase: first row of this wave's blocks within the tile.
  __device__ __forceinline__ void setup_reader(int rbase, int lane) {
    row0 = rbase + lane % CF::BLK;
    q = lane / CF::BLK;
  }

  // Instruction Q of K tile k_tile into the stage at LDS byte address sbase
  // (plus this wave's KiB).  GUARD: kvalid = bytes of K left from the tile's
  // start (> 0); chunks at or past it read as zero.  Without GUARD the K
  // tile is whole.
  template <int Q, bool GUARD>
  __device__ __forceinline__ void issue_one(uint32_t sbase, int k_tile, int kvalid) {
    uint32_t vo = voff;
    if constexpr (GUARD) vo = (int)cb < kvalid ? vo : 0x80000000u;
    dma16s<(uint32_t)Q * CF::NW * 1024u>(rsrc, sbase, vo, (uint32_t)k_tile * (uint32_t)CF::ROWB + Q * qstep);
  }

  // Fragment of MFMA block blk, k step s, from the stage at byte offset off
  // of the LDS array: lane group q's share (BPL bytes) of the step in row
  // row0 + blk*BLK.  Rows BLK apart share their chunk swizzle (a block spans
  // whole swizzle periods), so block blk is an immediate offset from block
  // 0's address.
  __device__ __forceinline__ typename CF::RAW read(const char* lds, int off, int blk, int s) const {
    static_assert(CF::BLK % (CF::CH << CF::SWZ_SHIFT) == 0, "block rows span whole swizzle periods");
    const char* rp = lds + off + row0 * CF::ROWB + blk * (CF::BLK * CF::ROWB);
    const int sw = swz<CF>(row0);
    if constexpr (CF::CPL == 1) {
      const int c = s * (CF::MM::KSB / 16) + q;
      return *(const v4i*)(rp + ((c ^ sw) << 4));
    } else {
      static_assert(CF::CPL == 2, "one or two chunks per lane");
      const int c = s * (CF::MM::KSB / 16) + q * CF::CPL;
      const v4i lo = *(const v4i*)(rp + ((c ^ sw) << 4));
      const v4i hi = *(const v4i*)(rp + (((c + 1) ^ sw) << 4));
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

// ---------------------------------------------------------------------------
// MN-major operand (A 'M' or B 'N'): a stage is BK k-rows of R elements (RB
// bytes); the 16-byte chunk c of k-row k is stored at c ^ mn_swz(k).  The
// MFMA wants each lane's k values of one row (m or n) side by side: the
// gfx950 transposing LDS loads give exactly that.  Within each group of 16
// lanes, ds_read_b64_tr_b16 reads 4 k-rows of 16 elements (4 lanes per k-row,
// 4 consecutive elements each) and hands lane i element i of every k-row;
// ds_read_b64_tr_b8 does the same with 8 k-rows (2 lanes per k-row, 8 bytes
// each).  So a lane receives E = 8 / ES consecutive k of one row per read.
// Out-of-range rows read as zero: the buffer's extent ends at the end of K,
// and a chunk past M (N) gets an out-of-range offset.
// ---------------------------------------------------------------------------
template <class CF>
struct MNSwizzle {
  // XOR applied to the chunk index of k-row k, chosen so that the chunks
  // read by one half-wave (32 lanes, one LDS cycle of 8-byte reads) hit 16
  // distinct 16-byte bank groups of the 64-bank LDS:
  //   2-byte, 16x16 blocks: k-rows {0..3, 8..11} (+4), 2 chunks each;
  //   2-byte, 32x32 blocks: k-rows {0..3} (+4), 4 chunks each;
  //   1-byte, 16x16 blocks, 16 B per lane: k-rows {0..7, 16..23} (+8), 1 chunk;
  //   1-byte, 32x32 blocks: k-rows {0..7} (+8), 2 chunks each.
  static constexpr __host__ __device__ int of(int k) {
    if constexpr (CF::MM::ESIZE == 2)
      return CF::BLK == 16 ? 2 * ((k & 3) | ((k >> 1) & 4)) : 4 * (k & 3);
    else if constexpr (CF::BLK == 32)
      return 2 * (k & 7);
    else
      return (k & 7) | ((k >> 1) & 8);
  }
  static constexpr int MAX = 15;
  // of(k) == of(k + step) for every k
  static constexpr bool periodic(int step) {
    for (int k = 0; k < 256; ++k)
      if (of(k) != of(k + step)) return false;
    return true;
  }
};

template <class CF, int R, int WR>
struct MNMajorOperand {
  static constexpr int ES = CF::MM::ESIZE;
  static constexpr int BK = CF::BK;       // k per stage
  static constexpr int RB = R * ES;       // bytes of one k-row
  static constexpr int CPR = RB / 16;     // chunks per k-row
  static constexpr int RPI = 1024 / RB;   // k-rows per wave instruction
  static constexpr int NQ = BK / (RPI * CF::NW);
  static_assert(RPI * RB == 1024 && NQ * RPI * CF::NW == BK, "k-rows must split evenly over the waves");
  static_assert(CPR > MNSwizzle<CF>::MAX, "the swizzle stays inside a k-row");
  static constexpr int E = 8 / ES;              // k per lane and transposing read
  static constexpr int KPL = CF::BPL / ES;      // k per lane and step
  static constexpr int NR = KPL / E;            // transposing reads per fragment
  static constexpr int KK = CF::MM::KSB / ES;   // k per step
  static constexpr int NBLK = WR / CF::BLK;  // blocks of the reading wave along R
  // The swizzle of the k-rows of instruction i depends on i only through
  // i & 1 (instructions are NW*RPI k-rows apart, a multiple of 8), so two
  // per-lane offsets serve them all; the rest of the step is a scalar.
  static constexpr int NV = NQ < 2 ? NQ : 2;
  static_assert(MNSwizzle<CF>::periodic(2 * CF::NW * RPI), "two offset patterns cover every instruction");
  v4i rsrc;
  uint32_t voff[NV];
  uint32_t kstride;  // bytes of one K tile in global memory
  uint32_t qstep;    // bytes between instructions i and i + 2
  int raddr;         // reader: LDS byte offset of block 0 (k step 0, read 0)

  // A K slice other than the last is a whole number of K tiles, so every
  // k-row staged from it lies inside it; k-rows past K read as zero.
  __device__ __forceinline__ void setup(const char* batch, int64_t extent, int64_t K, int64_t kbeg, int r0,
                                        int wave, int lane) {
    const int64_t ldb = extent * ES;  // bytes of one global k-row
    rsrc = make_rsrc(batch + (int64_t)r0 * ES + kbeg * ldb, (uint32_t)((K - kbeg) * ldb - (int64_t)r0 * ES));
    kstride = (uint32_t)(BK * ldb);
    qstep = (uint32_t)(2 * CF::NW * RPI * ldb);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int krow = (i * CF::NW + wave) * RPI + lane / CPR;
      const int lc = (lane % CPR) ^ MNSwizzle<CF>::of(krow);
      voff[i] = (int64_t)r0 + lc * (16 / ES) < extent ? (uint32_t)(krow * ldb + lc * 16) : 0x80000000u;
    }
  }
  // Block blk's chunks are block 0's with the bits of blk * BLK * ES flipped:
  // the row offset of the wave (a multiple of its WR rows), the block and the
  // lane's place inside a block occupy disjoint bits, and the swizzle is an
  // XOR, so the byte address of block blk is raddr ^ (blk * BLK * ES).
  __device__ __forceinline__ void setup_reader(int rbase, int lane) {
    static_assert((WR & (WR - 1)) == 0 && (CF::BLK * NBLK) == WR, "wave rows a power of two");
    constexpr int LPR = 16 / E;  // lanes per k-row in one read
    const int i16 = lane & 15, b = lane >> 4;
    const int q = CF::BLK == 16 ? b : b >> 1;           // k group of this lane
    const int roff = CF::BLK == 16 ? 0 : (b & 1) * 16;  // rows of the block's half
    const int krow = q * KPL + i16 / LPR;               // + s*KK + h*E at read time
    const int rbyte = (rbase + roff + (i16 % LPR) * E) * ES;
    raddr = krow * RB + (((rbyte >> 4) ^ MNSwizzle<CF>::of(krow)) << 4) + (rbyte & 15);
  }
  template <int Q, bool GUARD>
  __device__ __forceinline__ void issue_one(uint32_t sbase, int k_tile, int) {
    dma16s<(uint32_t)Q * CF::NW * 1024u>(rsrc, sbase, voff[Q & 1], (uint32_t)k_tile * kstride + (Q >> 1) * qstep);
  }

  // Fragment of block blk, k step s: NR transposing reads of E k each (the
  // swizzle of a lane's k-rows does not change with s or the read index).
  __device__ __forceinline__ typename CF::RAW read(const char* lds, int off, int blk, int s) const {
    lds_char_t* base = (lds_char_t*)lds + off + (raddr ^ (blk * CF::BLK * ES)) + s * KK * RB;
    int r[2 * NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      v2i v;
      if constexpr (ES == 2)
        v = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) v4s*)(base + h * E * RB)));
      else
        v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(base + h * E * RB));
      r[2 * h] = v.x;
      r[2 * h + 1] = v.y;
    }
    if constexpr (NR == 2) return v4i{r[0], r[1], r[2], r[3]};
    else return v8i{r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]};
  }
};

// R: rows of the operand tile (BM or BN); WR: rows of one wave's share.
template <class CF, int R, int WR, bool KMAJ>
using Operand = typename std::conditional<KMAJ, KMajorOperand<CF, R, WR>, MNMajorOperand<CF, R, WR>>::type;


// Accumulator element as the 32-bit pattern stored in LDS.  (The element is
// read into a scalar first: bit-casting a vector-element lvalue directly
// reads element 0 with this compiler.)
__device__ __forceinline__ float acc_bits(float v) { return v; }
__device__ __forceinline__ float acc_bits(int v) { return __int_as_float(v); }

// Writes 32-line block `blk` of this wave's accumulator tile into its LDS
// region (fp32 or int32 bit patterns): for N-major outputs rows blk*32 ..
// blk*32+31 of the wave tile (line = row, WN columns), for M-major columns
// (line = column, WM rows).
template <class CF, bool NMAJ, class ACC>
__device__ __forceinline__ void epi_stage_block(const ACC (&acc)[CF::FM][CF::FN], float* region, int lane,
                                                int blk) {
  using MM = typename CF::MM;
  constexpr int BLK = CF::BLK, PITCH = CF::epi_pitch(NMAJ), SUB = 32 / BLK;
  const int lc = lane % BLK;
  if constexpr (NMAJ) {
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

template <class CF, bool NMAJ, int T, bool UNIT = false, class ACC>
__device__ __forceinline__ void epilogue_typed(const Params& p, const ACC (&acc)[CF::FM][CF::FN], char* lds,
                                               int wave, int lane, int l, int mw, int nw) {
  constexpr int LINE = CF::epi_line(NMAJ), PITCH = CF::epi_pitch(NMAJ);
  constexpr int ES = EpiElem<T>::SIZE;
  constexpr int VEC = 16 / ES;         // elements per lane: one 16-byte access per array
  constexpr int LPL = LINE / VEC;      // lanes per line
  constexpr int LINES_PER_PASS = 64 / LPL;
  static_assert(LPL >= 1 && LPL <= 64 && 32 % LINES_PER_PASS == 0, "line split over the lanes");
  float* region = (float*)(lds + wave * CF::epi_wave_bytes(NMAJ));
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

  auto write_block = [&](auto blk_c) { epi_stage_block<CF, NMAJ>(acc, region, lane, decltype(blk_c)::value); };

  // Absent arrays read as zero (C, X) or are not written (Y) through empty
  // resources, except in the common form without X and Y: there the passes
  // run in a copy that issues no X loads and no Y stores at all, since even
  // accesses to an empty resource occupy the memory pipeline.  Both copies
  // are free of branches.
  auto passes = [&](auto xy_c) {
    constexpr bool XY = decltype(xy_c)::value != 0;
    v4u cr[DIST + 1], xr[DIST + 1];
    static_for<0, DIST>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      cr[i] = epi_ld<T>(rc, off(i));
      xr[i] = XY ? epi_ld<T>(rx, off(i)) : v4u{};
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
        xr[SN] = XY ? epi_ld<T>(rx, off(i + DIST)) : v4u{};
      }
      const uint32_t o = off(i);
      if constexpr (T == T_I32) {
        const v4u a = __builtin_bit_cast(v4u, w0);
        // UNIT: the scalars are 1 or their terms read zero (int_unit)
        v4u t = UNIT ? a + cr[S] : a * (unsigned)p.ialpha + cr[S] * (unsigned)p.ibeta;
        if (p.relu) t = relu4(t);
        t += UNIT ? xr[S] : xr[S] * (unsigned)p.ix;
        epi_st<T>(rd, o, t);
        if constexpr (XY) epi_st<T>(ry, o, a);
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
        if constexpr (XY) epi_st<T>(ry, o, epi_pack<T>(w0, w1));
      }
      // passes stay in program order: each issues its loads DIST passes ahead
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  if (p.X || p.Y) passes(IntC<1>{});
  else passes(IntC<0>{});
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

template <class CF, bool NMAJ, class ACC>
__device__ __forceinline__ void epilogue_mixed(const Params& p, const ACC (&acc)[CF::FM][CF::FN], char* lds,
                                               int wave, int lane, int l, int mw, int nw) {
  constexpr int LINE = CF::epi_line(NMAJ), PITCH = CF::epi_pitch(NMAJ);
  constexpr int VEC = 4;
  constexpr int LPL = LINE / VEC;
  constexpr int LINES_PER_PASS = 64 / LPL;
  static_assert(LPL >= 1 && LPL <= 64 && 32 % LINES_PER_PASS == 0, "line split over the lanes");
  float* region = (float*)(lds + wave * CF::epi_wave_bytes(NMAJ));
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

  auto write_block = [&](auto blk_c) { epi_stage_block<CF, NMAJ>(acc, region, lane, decltype(blk_c)::value); };

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

// uint8: the accumulator of each output of this wave's tile starts at
// 128*(rsum_a[m] + rsum_b[n]) + u8_bias (see Params).  The sums are loaded
// before the prologue's DMA (their wait is the prologue's) and applied after
// it, before any fragment is live.  Rows and columns past the matrix read
// zero through the buffers' range check; their outputs are never stored.
template <class CF>
struct U8Init {
  using MM = typename CF::MM;
  static constexpr int BLK = CF::BLK, ACCN = MM::ACCN, G = ACCN / 4;
  uint32_t cb[CF::FN];
  v4u rr[CF::FM][G];  // four consecutive rows per accumulator register group

  __device__ __forceinline__ void load(const Params& p, int l, int mw, int nw, int lane) {
    // resources based at this wave's first row / column; per-lane offsets
    // are one register each plus compile-time immediates
    // (a wave whose first row or column lies past the matrix gets an empty
    // resource: all its loads read zero)
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.rsum_a + (int64_t)l * p.M + mw), (short)0, (int)(max(p.M - mw, (int64_t)0) * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.rsum_b + (int64_t)l * p.N + nw), (short)0, (int)(max(p.N - nw, (int64_t)0) * 4), 0x00020000);
    const int la = MM::acc_row(lane, 0) * 4, lb = (lane % BLK) * 4;
#pragma unroll
    for (int j = 0; j < CF::FN; ++j) cb[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, lb + j * BLK * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g)
        rr[i][g] = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(
                     ra, la + (i * BLK + MM::acc_row(0, 4 * g) - MM::acc_row(0, 0)) * 4, 0, 0));
  }
  template <class ACC>
  __device__ __forceinline__ void apply(ACC (&acc)[CF::FM][CF::FN], int32_t bias) const {
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j)
#pragma unroll
        for (int v = 0; v < ACCN; ++v)
          acc[i][j][v] = (int)((rr[i][v / 4][v % 4] + cb[j]) * 128u + (uint32_t)bias);
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

  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int g = p.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  using OpA = Operand<CF, BM, CF::WM, CF::A_KMAJOR>;
  using OpB = Operand<CF, BN, CF::WN, CF::B_KMAJOR>;
  // DMA instructions per wave per stage (for the counted waits)
  constexpr int NQ_A = OpA::NQ;
  constexpr int NQ_STAGE = NQ_A + OpB::NQ;
  // LDS: A's stages, then B's stages.
  constexpr int A_STAGE = BM * CF::ROWB, B_STAGE = BN * CF::ROWB;
  constexpr int B_REGION = S * A_STAGE;

  OpA opa;
  OpB opb;
  opa.setup_reader(wm * CF::WM, lane);
  opb.setup_reader(wn * CF::WN, lane);
  using raw_t = typename CF::RAW;

  for (int t = g; t < p.tiles_total; t += G) {
    // ---- work item: a whole tile, or K slice `split` of tile ts ----------
    int split = -1;  // whole K range, epilogue here
    int ts = t;
    if (t >= p.dp_tiles) {
      const int u = t - p.dp_tiles;  // the item's workspace slot
      split = (int)((unsigned)u / (unsigned)p.tail_tiles);
      ts = p.dp_tiles + (u - split * p.tail_tiles);
    }
    const TileRC tc = raster_tile(ts, p.tiles_m, p.tiles_n, p.group_m);
    const int l = tc.l;
    const int64_t kbeg = split > 0 ? (int64_t)split * p.kslice : 0;
    const int64_t kbytes = (split < 0 ? p.K : min(p.K - kbeg, p.kslice)) * ES;  // this item's K, in bytes
    const int KT = (int)((kbytes + CF::ROWB - 1) / CF::ROWB);
    const int m0 = tc.tm * BM, n0 = tc.tn * BN;

    // ---- staging set-up --------------------------------------------------
    opa.setup((const char*)p.A + (int64_t)l * p.M * p.K * ES, p.M, p.K, kbeg, m0, wave, lane);
    opb.setup((const char*)p.B + (int64_t)l * p.N * p.K * ES, p.N, p.K, kbeg, n0, wave, lane);

    acc_t acc[CF::FM][CF::FN];
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) acc[i][j] = acc_t{};
    [[maybe_unused]] U8Init<CF> u8i;
    if constexpr (CF::U8) u8i.load(p, l, m0 + wm * CF::WM, n0 + wn * CF::WN, lane);

    // Fragments of one k step as read from LDS: A blocks then B blocks of
    // this wave (double-buffered).
    raw_t fa[2][CF::FM], fb[2][CF::FN];
    auto load_step = [&](raw_t (&ra)[CF::FM], raw_t (&rb)[CF::FN], int st, int s) {
#pragma unroll
      for (int i = 0; i < CF::FM; ++i) ra[i] = opa.read(lds, st * A_STAGE, i, s);
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) rb[j] = opb.read(lds, B_REGION + st * B_STAGE, j, s);
    };
    static_assert(CF::KSTEPS % 2 == 0, "k steps alternate fragment buffers across K tiles");

    // ---- explicitly ordered k steps ----------------------------------------
    // Each k step issues its MFMAs in a fixed order (sched_barrier pins it);
    // after each MFMA come the fragment reads of the next step scheduled
    // there (ordered by first use: A0, B0.., A1..) and a share of the DMA
    // instructions of a later K tile, so LDS reads, DMA and MFMAs overlap.
    constexpr int NREAD = CF::FM + CF::FN;
    constexpr int MF = CF::FM * CF::FN;
    auto read_r = [&](auto buf_c, auto r_c, auto st_x, auto ks_x) {
      constexpr int BUF = decltype(buf_c)::value, R = decltype(r_c)::value;
      const int st = (int)st_x, ks = (int)ks_x;
      if constexpr (R == 0)
        fa[BUF][0] = opa.read(lds, st * A_STAGE, 0, ks);
      else if constexpr (R <= CF::FN)
        fb[BUF][R - 1] = opb.read(lds, B_REGION + st * B_STAGE, R - 1, ks);
      else
        fa[BUF][R - CF::FN] = opa.read(lds, st * A_STAGE, R - CF::FN, ks);
    };
    // DMA instruction D of K tile k_tile into stage stg.  GUARD: the tile
    // may not exist (k_tile >= KT) or may be cut by the end of K; without
    // it the tile is whole and no check is made.
    const uint32_t lds_wave = lds_u32 + (uint32_t)wave * 1024u;
    auto dma_one = [&](auto d_c, auto guard_c, int k_tile, int stg) {
      constexpr int D = decltype(d_c)::value;
      constexpr bool GUARD = decltype(guard_c)::value;
      if (GUARD && k_tile >= KT) return;
      const int kv = GUARD ? (int)min(kbytes - (int64_t)k_tile * CF::ROWB, (int64_t)CF::ROWB) : CF::ROWB;
      if constexpr (D < NQ_A)
        opa.template issue_one<D, GUARD>(lds_wave + (uint32_t)stg * (uint32_t)A_STAGE, k_tile, kv);
      else
        opb.template issue_one<D - NQ_A, GUARD>(lds_wave + (uint32_t)(B_REGION + stg * B_STAGE), k_tile, kv);
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

    // Prologue: two stages: K tiles 0 and 1 whole, tile 0 complete.  Deep
    // ring: K tiles 0 .. S-2 whole, tile 0 complete, then part 0 of tile
    // S-1 (stage S-1 is untouched so far).
    // (tile numbers known at compile time are hidden from constant folding:
    // the DMA's scalar offset operand takes no literal)
    auto issue_tile = [&](int k_tile) {
      asm("" : "+s"(k_tile));
      static_for<0, NQ_STAGE>([&](auto d_c) { dma_one(d_c, IntC<1>{}, k_tile, k_tile % S); });
    };
    if constexpr (S == 2) {
      issue_tile(0);
      if (1 < KT) {
        issue_tile(1);
        wait_vmcnt<NQ_STAGE>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
#pragma unroll
      for (int k = 0; k < S - 1; ++k)
        if (k < KT) issue_tile(k);
      wait_pending(min(S - 1, KT) - 1);
      int t_pro = S - 1;
      asm("" : "+s"(t_pro));
      static_for<0, P0>([&](auto d_c) { dma_one(d_c, IntC<1>{}, t_pro, S - 1); });
    }
    barrier_lds();
    if constexpr (CF::U8) u8i.apply(acc, p.u8_bias);
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
    barrier_lds();  // every wave is done reading the ring

    // ---- fused epilogue ---------------------------------------------------
    // One element type for every C/X/D/Y in use and that type fp16 (8
    // elements per lane), fp32 or int32 (4): the one-type epilogue;
    // otherwise (bf16 included) the mixed-type one (4 elements per lane).
    constexpr bool NM = CF::CD_NMAJOR;
    const int emw = m0 + wm * CF::WM, enw = n0 + wn * CF::WN;
    if (t >= p.dp_tiles) {
      // a K slice: its partial sums, unscaled, into its workspace slot, as a
      // rows x cols matrix of its own (the tile's part inside the matrix)
      Params q = p;
      q.D = (char*)p.ws + (int64_t)(t - p.dp_tiles) * (BM * BN * 4);
      q.M = min(p.M - m0, (int64_t)BM);
      q.N = min(p.N - n0, (int64_t)BN);
      q.L = 1;
      q.C = q.X = nullptr;
      q.Y = nullptr;
      q.alpha = 1.0f;
      q.beta = q.xf = 0.0f;
      q.ialpha = 1;
      q.ibeta = q.ix = 0;
      q.relu = 0;
      if constexpr (CF::INT) epilogue_typed<CF, NM, T_I32, true>(q, acc, lds, wave, lane, 0, emw - m0, enw - n0);
      else epilogue_typed<CF, NM, T_F32>(q, acc, lds, wave, lane, 0, emw - m0, enw - n0);
    } else if constexpr (CF::INT) {
      if (p.int_unit) epilogue_typed<CF, NM, T_I32, true>(p, acc, lds, wave, lane, l, emw, enw);
      else epilogue_typed<CF, NM, T_I32, false>(p, acc, lds, wave, lane, l, emw, enw);
    } else {
      if (p.epi_kind == T_F16) epilogue_typed<CF, NM, T_F16>(p, acc, lds, wave, lane, l, emw, enw);
      else if (p.epi_kind == T_F32) epilogue_typed<CF, NM, T_F32>(p, acc, lds, wave, lane, l, emw, enw);
      else epilogue_mixed<CF, NM>(p, acc, lds, wave, lane, l, emw, enw);
    }
    barrier_lds();  // LDS is reused by the next tile's prologue
  }
}

}  // namespace gemm_epi
