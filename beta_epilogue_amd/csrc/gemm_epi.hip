// gemm_epi.hip -- C ABI of the fused-epilogue batched GEMM (see
// include/gemm_epi.h): validation, variant choice, persistent launch.
//
// Conventions follow the Blackwell pipeline API card ("Host side": a plan is
// built once and checked before launch, errors come back as codes with a
// string function; "Device side": one handle serves the whole persistent
// grid) and the "Constraints" of the CuTe DSL example
// custom_epilogue_dense_gemm.py (A/B share a type, C/D/X/Y share a
// majorness, contiguous extents are 16-byte multiples).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "gemm_epi.h"
#include "gemm_epi_kernel.hpp"
#include "gemm_epi_launch.hpp"
#include "gemm_epi_splitk.hpp"
#include "gemm_epi_prep.hpp"

namespace {

thread_local char g_last_error[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

using gemm_epi::Params;
typedef void (*launch_fn)(const Params&, int grid, hipStream_t s);

struct Variant {
  const char* name;
  int ab;          // A/B element type
  int a_major;     // GEMM_EPI_MAJOR_*
  int b_major;
  int cd_major;
  int bm, bn, bk, threads, lds;
  int blk;         // MFMA output block (16 or 32)
  launch_fn launch;
};


template <class CF>
constexpr Variant make_variant(const char* name) {
  return Variant{name,
                 CF::AB,
                 CF::A_KMAJOR ? GEMM_EPI_MAJOR_K : GEMM_EPI_MAJOR_M,
                 CF::B_KMAJOR ? GEMM_EPI_MAJOR_K : GEMM_EPI_MAJOR_N,
                 CF::CD_NMAJOR ? GEMM_EPI_MAJOR_N : GEMM_EPI_MAJOR_M,
                 CF::BM,
                 CF::BN,
                 CF::BK,
                 CF::THREADS,
                 CF::LDS_BYTES,
                 CF::BLK,
                 &gemm_epi::launch<CF>};
}

using namespace gemm_epi;
// Variant table (gemm_epi_variants.inc); the kernels are compiled in the
// gemm_epi_part.hip translation units, this one only refers to them.
#define X(PART, AB, AK, BK, CDN, BM, BN, RB, WM, WN, S, DS, BL, NAME) \
  make_variant<Cfg<AB, AK, BK, CDN, BM, BN, RB, WM, WN, S, DS, BL>>(NAME),
const Variant kVariants[] = {
#include <gemm_epi_variants.inc>  // (angle brackets: a partial build can put its own table first)
};
#undef X
#undef V
#undef VR
#undef VD
constexpr int kNumVariants = (int)(sizeof kVariants / sizeof kVariants[0]);

int elem_bytes(int t) {
  switch (t) {
    case GEMM_EPI_F16:
    case GEMM_EPI_BF16: return 2;
    case GEMM_EPI_E4M3:
    case GEMM_EPI_E5M2:
    case GEMM_EPI_I8:
    case GEMM_EPI_U8: return 1;
    case GEMM_EPI_F32:
    case GEMM_EPI_I32: return 4;
    default: return 0;
  }
}

bool is_float_out(int t) { return t == GEMM_EPI_F16 || t == GEMM_EPI_BF16 || t == GEMM_EPI_F32; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

}  // namespace

// The uint8 workspace: sums of A rows (L*M int32) and of B columns (L*N),
// then the flipped copies of A (L*M*K bytes) and B (L*N*K), each part at a
// 256-byte boundary.  Returns its size; with base set, the parts' addresses.
static int64_t u8_layout(const gemm_epi_desc* d, char* base, int32_t** sums, uint8_t** flipped) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t sums_bytes = up(d->L * (d->M + d->N) * 4);
  const int64_t a_bytes = up(d->L * d->M * d->K);
  const int64_t b_bytes = up(d->L * d->N * d->K);
  if (base) {
    *sums = (int32_t*)base;
    flipped[0] = (uint8_t*)base + sums_bytes;
    flipped[1] = (uint8_t*)base + sums_bytes + a_bytes;
  }
  return sums_bytes + a_bytes + b_bytes;
}

struct gemm_epi_handle {
  gemm_epi_desc desc;
  int variant;
  int grid;
  int cus;
  int device;
  int64_t tiles_m, tiles_n, tiles;  // output tiles (one K slice)
  int group_m;
  int splits;                       // K slices of a split tile (1: no split)
  int64_t kslice;                   // K elements per slice
  int64_t dp_tiles, tail_tiles;     // whole tiles first, then the split ones
  int64_t items;                    // work items: dp_tiles + tail_tiles * splits
  int64_t ws_bytes;                 // workspace: split-K partial sums, then the prepared operands
  bool widen;                       // fp8 A/B run as fp16 copies
  int64_t prep_off;                 // the prepared operands (uint8 sums and copies, fp16 copies)
  std::atomic<void*> ws{nullptr};   // allocated by the first gemm_epi_run, freed by destroy
  std::mutex ws_mutex;
  void* ws_static = nullptr;        // device address of the static scratch array
};

// ---------------------------------------------------------------------------
// Allocation-free runs (gemm_epi_run_static): the split-K workspace is a
// file-scope device array, one copy per GPU, instead of memory of the handle.
// Host code uses the array's device address from hipGetSymbolAddress (taken
// once per device, with that device current), never the array's name.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = GEMM_EPI_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (NULL: not taken yet)

// The device address of `scratch` on the current device `dev`.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(GEMM_EPI_ERR_DEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GEMM_EPI_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_EPI_OK;
}
}  // namespace

// Static validation: everything that needs no device.
static int validate_desc(const gemm_epi_desc* d) {
  if (!d) return fail(GEMM_EPI_ERR_INVALID_ARG, "desc is NULL");
  if (d->M < 1 || d->N < 1 || d->K < 1 || d->L < 1)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "M, N, K, L must be >= 1 (got %lld %lld %lld %lld)",
                (long long)d->M, (long long)d->N, (long long)d->K, (long long)d->L);
  int64_t mk, nk, mn, t;
  if (!mul_ok(d->M, d->K, &mk) || !mul_ok(mk, d->L, &t) || !mul_ok(d->N, d->K, &nk) ||
      !mul_ok(nk, d->L, &t) || !mul_ok(d->M, d->N, &mn) || !mul_ok(mn, d->L, &t) ||
      !mul_ok(t, 4, &t))
    return fail(GEMM_EPI_ERR_INVALID_ARG, "tensor byte sizes overflow int64");
  if (d->a_major != GEMM_EPI_MAJOR_K && d->a_major != GEMM_EPI_MAJOR_M)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "a_major must be K or M");
  if (d->b_major != GEMM_EPI_MAJOR_K && d->b_major != GEMM_EPI_MAJOR_N)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "b_major must be K or N");
  if (d->cd_major != GEMM_EPI_MAJOR_N && d->cd_major != GEMM_EPI_MAJOR_M)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "cd_major must be N or M");
  if (d->b_dtype != GEMM_EPI_NONE && d->b_dtype != d->ab_dtype &&
      !((d->ab_dtype == GEMM_EPI_E4M3 || d->ab_dtype == GEMM_EPI_E5M2) &&
        (d->b_dtype == GEMM_EPI_E4M3 || d->b_dtype == GEMM_EPI_E5M2)))
    return fail(GEMM_EPI_ERR_INVALID_ARG, "b_dtype may differ from ab_dtype only as the other fp8 format");
  if (d->splits < 0) return fail(GEMM_EPI_ERR_INVALID_ARG, "splits must be >= 0 (got %d)", d->splits);
  if (d->epilogue != GEMM_EPI_LINEAR && d->epilogue != GEMM_EPI_RELU)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "epilogue must be LINEAR or RELU (got %d)", d->epilogue);
  const int ab = d->ab_dtype;
  if (ab != GEMM_EPI_F16 && ab != GEMM_EPI_BF16 && ab != GEMM_EPI_E4M3 && ab != GEMM_EPI_E5M2 &&
      ab != GEMM_EPI_I8 && ab != GEMM_EPI_U8)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "ab_dtype must be F16, BF16, E4M3, E5M2, I8 or U8");
  const bool int_path = ab == GEMM_EPI_I8 || ab == GEMM_EPI_U8;
  auto out_ok = [&](int t, bool allow_none) {
    if (t == GEMM_EPI_NONE) return allow_none;
    return int_path ? t == GEMM_EPI_I32 : is_float_out(t);
  };
  for (int t : {d->c_dtype, d->x_dtype, d->d_dtype, d->y_dtype})
    if (t < GEMM_EPI_NONE || t > GEMM_EPI_U8)
      return fail(GEMM_EPI_ERR_INVALID_ARG, "unknown dtype code %d", t);
  if (!out_ok(d->c_dtype, true) || !out_ok(d->x_dtype, true) || !out_ok(d->d_dtype, false) ||
      !out_ok(d->y_dtype, true))
    return fail(GEMM_EPI_ERR_UNSUPPORTED,
                int_path ? "int8/uint8 A/B need int32 C/X/D/Y (D required)"
                         : "float A/B need F16/BF16/F32 C/X/D/Y (D required)");
  // 16-byte rule on the contiguous extent of every tensor.
  const int es = elem_bytes(ab);
  const int64_t a_contig = d->a_major == GEMM_EPI_MAJOR_K ? d->K : d->M;
  const int64_t b_contig = d->b_major == GEMM_EPI_MAJOR_K ? d->K : d->N;
  if ((a_contig * es) % 16 || (b_contig * es) % 16)
    return fail(GEMM_EPI_ERR_ALIGNMENT,
                "contiguous extent of A (%lld) and B (%lld) must be a multiple of 16 bytes",
                (long long)a_contig, (long long)b_contig);
  const int64_t cd_contig = d->cd_major == GEMM_EPI_MAJOR_N ? d->N : d->M;
  for (int t : {d->c_dtype, d->x_dtype, d->d_dtype, d->y_dtype})
    if (t != GEMM_EPI_NONE && (cd_contig * elem_bytes(t)) % 16)
      return fail(GEMM_EPI_ERR_ALIGNMENT,
                  "contiguous extent %lld of C/X/D/Y is not a multiple of 16 bytes",
                  (long long)cd_contig);
  return GEMM_EPI_OK;
}

// A/B types of a problem: A's, and B's (A's unless an fp8 pair).
static int b_type(const gemm_epi_desc* d) { return d->b_dtype == GEMM_EPI_NONE ? d->ab_dtype : d->b_dtype; }
static bool is_fp8(int t) { return t == GEMM_EPI_E4M3 || t == GEMM_EPI_E5M2; }

// The kernel code of a problem: the common type (uint8: the int8 kernels on
// flipped copies, accumulators started at the sums' correction) or an fp8
// pair.
static int exact_ab(const gemm_epi_desc* d) {
  const int a = d->ab_dtype, b = b_type(d);
  if (a == GEMM_EPI_U8 && b == GEMM_EPI_U8) return gemm_epi::T_U8;
  if (a == b) return a;
  if (a == GEMM_EPI_E4M3 && b == GEMM_EPI_E5M2) return gemm_epi::T_E4M3_E5M2;
  if (a == GEMM_EPI_E5M2 && b == GEMM_EPI_E4M3) return gemm_epi::T_E5M2_E4M3;
  return -1;
}

static bool same_layout(const Variant& v, const gemm_epi_desc* d) {
  return v.a_major == d->a_major && v.b_major == d->b_major && v.cd_major == d->cd_major;
}

// fp8 A/B that run widened: a preparation pass converts A and B to fp16
// copies (exact: every e4m3 and e5m2 value is an fp16 value) and an fp16
// kernel of the same layout runs on them.  So it is for an fp32 D or Y (the
// fp8 MFMA sums a group of products with fewer fraction bits than fp32
// keeps) and for the pairings and layouts no fp8-MFMA kernel is built for.
static bool widened(const gemm_epi_desc* d) {
  if (!is_fp8(d->ab_dtype) || !is_fp8(b_type(d))) return false;
  if (d->d_dtype == GEMM_EPI_F32 || d->y_dtype == GEMM_EPI_F32) return true;
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].ab == exact_ab(d) && same_layout(kVariants[i], d)) return false;
  return true;
}

// Whether variant v runs the problem: the layout's kernel of the problem's
// type, or of fp16 for a widened fp8 problem.
static bool variant_fits(const Variant& v, const gemm_epi_desc* d) {
  if (!same_layout(v, d)) return false;
  return v.ab == (widened(d) ? gemm_epi::T_F16 : exact_ab(d));
}

// Plan cost model (measured on MI355X, fp16 with C, X, D, Y; times in us).
// A K tile of one output tile takes 1.1 us with 256x256 tiles; with the
// smaller tiles their share of the work at a lower per-CU rate (192x256:
// 0.75 at 0.9, 128x256: 0.5 at 0.67, 128x128: 0.25 at ~0.46).  The split-K
// reduction costs 4 us plus its bytes (S partial-sum slots and C, X, D, Y
// per split tile) at 5 TB/s.
static double ktile_us(const Variant& v) {
  if (v.bm == 256 && v.bn == 256) return 1.1;
  if (v.bm == 192 && v.bn == 256) return 1.1 * 0.75 / 0.9;
  if (v.bm == 128 && v.bn == 256) return 1.1 * 0.75;
  return 0.6;
}

struct SplitChoice {
  int64_t splits, tail;  // K slices of the split tiles (1: none), split tiles
  double us;             // modelled time of the launch
};

// The library's split choice for variant v and the modelled time: when the
// last round of tiles (tiles % cus, all of them with fewer tiles than CUs)
// would leave at least half of the CUs idle, those tiles may run in S K
// slices after whole-K rounds of the others; S (2 .. min(cus / last,
// K tiles / 4, 16)) maximises the time saved in the last round,
// (K tiles - ceil(K tiles / S)) K-tile times, less the reduction's cost; no S
// with a positive balance, no split.
static SplitChoice split_choice(const Variant& v, const gemm_epi_desc* d, int64_t cus) {
  const int64_t tiles = ((d->M + v.bm - 1) / v.bm) * ((d->N + v.bn - 1) / v.bn) * d->L;
  const int64_t ktiles = (d->K + v.bk - 1) / v.bk;
  const double tk = ktile_us(v);
  const int64_t last = tiles % cus;
  SplitChoice c{1, 0, (double)((tiles + cus - 1) / cus) * ktiles * tk};
  if (last == 0 || last * 2 > cus || d->ab_dtype == GEMM_EPI_U8) return c;
  const double slot_bytes = 4.0 * v.bm * v.bn;
  double epi_bytes = 0.0;
  for (int t : {d->c_dtype, d->x_dtype, d->d_dtype, d->y_dtype})
    if (t != GEMM_EPI_NONE) epi_bytes += (double)elem_bytes(t) * v.bm * v.bn;
  const int64_t smax = std::min<int64_t>(std::min<int64_t>(cus / last, ktiles / 4), 16);
  double best = 0.0;
  for (int64_t s = 2; s <= smax; ++s) {
    const double saved_us = (double)(ktiles - (ktiles + s - 1) / s) * tk;
    const double cost_us = 4.0 + (double)last * (s * slot_bytes + epi_bytes) / 5.0e6;
    if (saved_us - cost_us > best) {
      best = saved_us - cost_us;
      c.splits = s;
    }
  }
  if (c.splits > 1) {
    c.tail = last;
    c.us -= best;
  }
  return c;
}

extern "C" int gemm_epi_create_variant(const gemm_epi_desc* desc, int variant,
                                       gemm_epi_handle** out) {
  g_last_error[0] = 0;
  if (!out) return fail(GEMM_EPI_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_desc(desc);
  if (rc) return rc;
  if (variant < -1 || variant >= kNumVariants)
    return fail(GEMM_EPI_ERR_INVALID_ARG, "variant %d out of range", variant);
  const bool auto_variant = variant == -1;
  if (variant == -1) {
    for (int i = 0; i < kNumVariants; ++i)
      if (variant_fits(kVariants[i], desc)) {
        variant = i;
        break;
      }
    if (variant == -1)
      return fail(GEMM_EPI_ERR_UNSUPPORTED,
                  "no kernel for this dtype/majorness combination (ab=%d a=%d b=%d cd=%d)",
                  desc->ab_dtype, desc->a_major, desc->b_major, desc->cd_major);
  } else if (!variant_fits(kVariants[variant], desc)) {
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "variant %s cannot run this problem",
                kVariants[variant].name);
  }
  const Variant* vp = &kVariants[variant];
  // Buffer offsets within one tile's rows are 32-bit (a widened fp8 operand
  // is read as its fp16 copy).
  const int es = widened(desc) ? 2 : elem_bytes(desc->ab_dtype);
  if ((int64_t)vp->bm * desc->K * es >= (int64_t(1) << 31) ||
      (int64_t)vp->bn * desc->K * es >= (int64_t(1) << 31))
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "K too large for 32-bit tile offsets");
  // An M-major A or N-major B is addressed with 32-bit offsets over all of K.
  const int64_t kpad = desc->K + 2 * (int64_t)vp->bk;
  if ((desc->a_major == GEMM_EPI_MAJOR_M && kpad * desc->M * es >= (int64_t(1) << 31)) ||
      (desc->b_major == GEMM_EPI_MAJOR_N && kpad * desc->N * es >= (int64_t(1) << 31)))
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "M-major A / N-major B larger than 2 GiB per batch");
  // The epilogue addresses a wave's output lines (at most a tile's BM or BN
  // lines of the leading extent) with 31-bit byte offsets.
  const int64_t ld = desc->cd_major == GEMM_EPI_MAJOR_N ? desc->N : desc->M;
  if ((int64_t)(vp->bm > vp->bn ? vp->bm : vp->bn) * ld * 4 >= (int64_t(1) << 31))
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "leading extent %lld of C/X/D/Y too long for 31-bit offsets",
                (long long)ld);
  // uint8: the row and column sums of a batch are addressed with 31-bit offsets.
  if (desc->ab_dtype == GEMM_EPI_U8 && (desc->M >= (int64_t(1) << 29) || desc->N >= (int64_t(1) << 29)))
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "uint8 needs M and N below 2^29");

  // Device query (the only part that needs a GPU).
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GEMM_EPI_ERR_DEVICE, "hipGetDevice failed");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(GEMM_EPI_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(GEMM_EPI_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev,
                prop.gcnArchName);

  // Tile shape (the library's choice, where the layout has the smaller
  // kernels: K-major A and B, N-major C/D).  128x128 tiles when the
  // 256x256 ones would fill at most a quarter of the CUs: four times the
  // tiles at about half the per-CU rate (fp16 with C, X, D, Y, TFLOP/s:
  // 1024^3 88 -> 193, 2048^3 366 -> 553, 2048^2 x 512 165 -> 346, 1024^2 x
  // 8192 428 -> 534).  Otherwise, when the 256x256 tiles leave a partial
  // round, the 192x256 or 128x256 plan with the lowest modelled time (its
  // own split choice included) if below 0.95 of the 256x256 plan's (3072^3
  // 718 -> 854 with 192x256, 2560^3 506 -> 675 and 2048 x 4096 x 4096
  // 774 -> 970 with 128x256; 4096^3, 3584^3 and 8192^3 keep 256x256).
  auto find_tile = [&](int bm, int bn) {
    for (int i = 0; i < kNumVariants; ++i)
      if (kVariants[i].bm == bm && kVariants[i].bn == bn && variant_fits(kVariants[i], desc)) return i;
    return -1;
  };
  if (auto_variant && desc->splits == 0) {
    const int64_t cus = prop.multiProcessorCount;
    const int64_t tiles_default =
        ((desc->M + vp->bm - 1) / vp->bm) * ((desc->N + vp->bn - 1) / vp->bn) * desc->L;
    const int small = find_tile(128, 128);
    if (small >= 0 && tiles_default * 4 <= cus) {
      variant = small;
    } else if (tiles_default % cus != 0) {
      double best = 0.95 * split_choice(*vp, desc, cus).us;
      for (const int cand : {find_tile(192, 256), find_tile(128, 256)}) {
        if (cand < 0) continue;
        const double t = split_choice(kVariants[cand], desc, cus).us;
        if (t < best) {
          best = t;
          variant = cand;
        }
      }
    }
    vp = &kVariants[variant];
  }
  const Variant& v = *vp;

  gemm_epi_handle* h = new (std::nothrow) gemm_epi_handle;
  if (!h) return fail(GEMM_EPI_ERR_HOST_ALLOC, "out of host memory");
  h->desc = *desc;
  h->variant = variant;
  h->device = dev;
  h->cus = prop.multiProcessorCount;
  h->tiles_m = (desc->M + v.bm - 1) / v.bm;
  h->tiles_n = (desc->N + v.bn - 1) / v.bn;
  h->tiles = h->tiles_m * h->tiles_n * desc->L;
  // Grouped raster: a workgroup's XCD takes 32 consecutive tiles, group_m
  // tile rows by 32 / group_m columns (4 x 8 or 8 x 4: 12 panels of A and B
  // either way); with more than 32 tile columns 8 rows also keep a round of
  // tiles nearer square (12288^3 fp16: +8 %; 8192^3 and narrower: equal).
  h->group_m = h->tiles_n > 32 ? 8 : 4;
  // Split K: the library's choice (split_choice, desc->splits == 0); uint8
  // never (its correction starts the accumulator of the whole K range);
  // desc->splits >= 2 splits every tile into that many slices.
  const int64_t ktiles = (desc->K + v.bk - 1) / v.bk;
  int64_t splits = 1, tail = 0;
  const bool u8 = desc->ab_dtype == GEMM_EPI_U8;
  if (u8) {
    splits = 1;
  } else if (desc->splits >= 1) {
    splits = std::min<int64_t>(desc->splits, ktiles);
    tail = h->tiles;
  } else {
    const SplitChoice c = split_choice(v, desc, h->cus);
    splits = c.splits;
    tail = c.tail;
  }
  if (splits < 1) splits = 1;
  h->kslice = ((ktiles + splits - 1) / splits) * v.bk;
  h->splits = (int)((desc->K + h->kslice - 1) / h->kslice);
  if (h->splits == 1) {
    h->kslice = desc->K;
    tail = 0;
  }
  h->tail_tiles = tail;
  h->dp_tiles = h->tiles - tail;
  // Workspace: the split-K partial sums, then (at a 256-byte boundary) the
  // prepared operands: for uint8 the row sums of A, the column sums of B and
  // the flipped copies of A and B, for widened fp8 the fp16 copies of A and
  // B (each part at a 256-byte boundary).
  h->widen = widened(desc);
  h->ws_bytes = h->splits > 1 ? (int64_t)h->splits * h->tail_tiles * v.bm * v.bn * 4 : 0;
  h->prep_off = (h->ws_bytes + 255) / 256 * 256;
  if (u8) h->ws_bytes = h->prep_off + u8_layout(desc, nullptr, nullptr, nullptr);
  if (h->widen)
    h->ws_bytes = h->prep_off + (desc->L * desc->M * desc->K * 2 + 255) / 256 * 256 +
                  (desc->L * desc->N * desc->K * 2 + 255) / 256 * 256;
  h->items = h->dp_tiles + h->tail_tiles * h->splits;
  if (h->items >= ((int64_t)1 << 31)) {
    const long long items = (long long)h->items;
    delete h;
    return fail(GEMM_EPI_ERR_UNSUPPORTED, "%lld work items (tiles and K slices): at most 2^31 - 1", items);
  }
  h->grid = (int)std::min<int64_t>(h->items, (int64_t)h->cus);  // one workgroup per CU
  if (scratch_address(dev, &h->ws_static) != GEMM_EPI_OK) {
    delete h;
    return GEMM_EPI_ERR_DEVICE;
  }
  *out = h;
  return GEMM_EPI_OK;
}

extern "C" int gemm_epi_create(const gemm_epi_desc* desc, gemm_epi_handle** out) {
  return gemm_epi_create_variant(desc, -1, out);
}

static bool integral_24(float v) {
  return std::isfinite(v) && std::nearbyint(v) == v && std::fabs(v) <= 16777216.0f;
}

// One fused GEMM; split-K plans use the handle's workspace (allocated here on
// first use) or, with use_static, the static scratch array.
static int run_impl(const gemm_epi_handle* hc, const void* A, const void* B, const void* C, const void* X,
                    void* D, void* Y, float alpha, float beta, float x_factor, void* stream, bool use_static) {
  g_last_error[0] = 0;
  if (!hc) return fail(GEMM_EPI_ERR_INVALID_ARG, "handle is NULL");
  gemm_epi_handle* h = const_cast<gemm_epi_handle*>(hc);  // only the lazily allocated workspace changes
  const gemm_epi_desc& d = h->desc;
  if (!A || !B || !D) return fail(GEMM_EPI_ERR_INVALID_ARG, "A, B and D are required");
  const bool use_c = d.c_dtype != GEMM_EPI_NONE && beta != 0.0f;
  const bool use_x = d.x_dtype != GEMM_EPI_NONE && x_factor != 0.0f;
  if (use_c && !C) return fail(GEMM_EPI_ERR_INVALID_ARG, "C is NULL but beta != 0");
  if (use_x && !X) return fail(GEMM_EPI_ERR_INVALID_ARG, "X is NULL but x_factor != 0");
  if ((d.y_dtype != GEMM_EPI_NONE) != (Y != nullptr))
    return fail(GEMM_EPI_ERR_INVALID_ARG, "Y must be given exactly when y_dtype is set");
  // In place: D may be C itself (same type); other shared pointers are errors.
  if (D == C && C && !(use_c && d.c_dtype == d.d_dtype))
    return fail(GEMM_EPI_ERR_INVALID_ARG, "D may alias C only when C is read and has D's dtype");
  if ((X && (D == X || Y == X)) || (Y && (Y == C || Y == D)))
    return fail(GEMM_EPI_ERR_INVALID_ARG, "outputs may not alias X, each other, or C (Y)");
  for (const void* ptr : {A, B, (const void*)D, use_c ? C : nullptr, use_x ? X : nullptr,
                          (const void*)Y})
    if (((uintptr_t)ptr) & 15u) return fail(GEMM_EPI_ERR_ALIGNMENT, "pointer %p is not 16-byte aligned", ptr);
  const bool u8 = d.ab_dtype == GEMM_EPI_U8;
  const bool int_path = d.ab_dtype == GEMM_EPI_I8 || u8;
  if (int_path && !(integral_24(alpha) && integral_24(beta) && integral_24(x_factor)))
    return fail(GEMM_EPI_ERR_UNSUPPORTED,
                "int32 outputs need integral alpha, beta, x_factor with |value| <= 2^24");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return fail(GEMM_EPI_ERR_DEVICE, "current device %d is not the handle's device %d", dev,
                h->device);

  Params p;
  p.A = A;
  p.B = B;
  p.C = use_c ? C : nullptr;
  p.X = use_x ? X : nullptr;
  p.D = D;
  p.Y = Y;
  p.M = d.M;
  p.N = d.N;
  p.K = d.K;
  p.tiles_total = (int32_t)h->items;
  p.L = (int32_t)d.L;
  p.tiles_m = (int32_t)h->tiles_m;
  p.tiles_n = (int32_t)h->tiles_n;
  p.group_m = h->group_m;
  p.c_dtype = use_c ? d.c_dtype : GEMM_EPI_NONE;
  p.x_dtype = use_x ? d.x_dtype : GEMM_EPI_NONE;
  p.d_dtype = d.d_dtype;
  p.y_dtype = d.y_dtype;
  p.alpha = alpha;
  p.beta = beta;
  p.xf = x_factor;
  p.ialpha = int_path ? (int32_t)alpha : 0;
  p.ibeta = int_path ? (int32_t)beta : 0;
  p.ix = int_path ? (int32_t)x_factor : 0;
  p.xcd_remap = (h->grid % 8 == 0) ? 1 : 0;
  p.relu = d.epilogue == GEMM_EPI_RELU ? 1 : 0;
  // Element type shared by every C/X/D/Y in use (one-type epilogue), else 0
  // (mixed-type epilogue).
  int kind = d.d_dtype;
  for (int t : {use_c ? d.c_dtype : 0, use_x ? d.x_dtype : 0, d.y_dtype})
    if (t != GEMM_EPI_NONE && t != kind) kind = 0;
  p.epi_kind = kind;
  p.dp_tiles = (int32_t)h->dp_tiles;
  p.tail_tiles = (int32_t)h->tail_tiles;
  p.splits = h->splits;
  p.kslice = h->kslice;
  p.ws = nullptr;
  p.rsum_a = p.rsum_b = nullptr;
  p.u8_bias = 0;
  p.int_unit = int_path && p.ialpha == 1 && (p.ibeta == 1 || !use_c) && (p.ix == 1 || !use_x) ? 1 : 0;
  if (h->ws_bytes > 0) {
    if (use_static) {
      if (h->ws_bytes > kScratchBytes)
        return fail(GEMM_EPI_ERR_UNSUPPORTED,
                    "workspace of %lld bytes exceeds the static scratch of %lld bytes",
                    (long long)h->ws_bytes, (long long)kScratchBytes);
      p.ws = h->ws_static;
    } else {
      p.ws = h->ws.load();
      if (!p.ws) {
        std::lock_guard<std::mutex> lock(h->ws_mutex);
        p.ws = h->ws.load();
        if (!p.ws) {
          if (hipMalloc(&p.ws, (size_t)h->ws_bytes) != hipSuccess || !p.ws)
            return fail(GEMM_EPI_ERR_DEVICE, "hipMalloc of a %lld-byte workspace failed",
                        (long long)h->ws_bytes);
          h->ws.store(p.ws);
        }
      }
    }
  }

  (void)hipGetLastError();  // clear a stale error so the check below is ours
  if (h->widen) {
    // fp16 copies of the fp8 operands (exact), read by the fp16 kernel
    uint16_t* wa = (uint16_t*)((char*)p.ws + h->prep_off);
    uint16_t* wb = (uint16_t*)((char*)wa + (d.L * d.M * d.K * 2 + 255) / 256 * 256);
    gemm_epi::launch_f8_widen((const uint8_t*)A, d.L * d.M * d.K, d.ab_dtype == GEMM_EPI_E5M2, wa,
                              (hipStream_t)stream);
    gemm_epi::launch_f8_widen((const uint8_t*)B, d.L * d.N * d.K, b_type(&d) == GEMM_EPI_E5M2, wb,
                              (hipStream_t)stream);
    p.A = wa;
    p.B = wb;
  }
  if (u8) {
    // one pass over each operand: its flipped copy (u - 128 as a signed
    // byte) and its sums along K; the GEMM reads the copies, and every
    // accumulator starts at 128 * (row sum + column sum) - 16384 * K
    int32_t* sums = nullptr;
    uint8_t* flipped[2] = {nullptr, nullptr};
    u8_layout(&d, (char*)p.ws + h->prep_off, &sums, flipped);
    int32_t* ra = sums;
    int32_t* rb = sums + d.L * d.M;
    gemm_epi::launch_u8_prep((const uint8_t*)A, d.a_major == GEMM_EPI_MAJOR_K, d.L, d.M, d.K, flipped[0], ra,
                             (hipStream_t)stream);
    gemm_epi::launch_u8_prep((const uint8_t*)B, d.b_major == GEMM_EPI_MAJOR_K, d.L, d.N, d.K, flipped[1], rb,
                             (hipStream_t)stream);
    p.A = flipped[0];
    p.B = flipped[1];
    p.rsum_a = ra;
    p.rsum_b = rb;
    p.u8_bias = (int32_t)(uint32_t)((uint64_t)(-(int64_t)16384 * d.K) & 0xffffffffu);
    p.ws = nullptr;
  }
  kVariants[h->variant].launch(p, h->grid, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GEMM_EPI_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  if (h->splits > 1) {
    // the slices' sums and the epilogue, on the same stream
    gemm_epi::SplitkParams q;
    q.ws = p.ws;
    q.C = p.C;
    q.X = p.X;
    q.D = D;
    q.Y = Y;
    q.M = d.M;
    q.N = d.N;
    q.dp_tiles = (int32_t)h->dp_tiles;
    q.tail_tiles = (int32_t)h->tail_tiles;
    q.tiles_m = (int32_t)h->tiles_m;
    q.tiles_n = (int32_t)h->tiles_n;
    q.group_m = h->group_m;
    q.tile_m = kVariants[h->variant].bm;
    q.tile_n = kVariants[h->variant].bn;
    q.cd_nmajor = d.cd_major == GEMM_EPI_MAJOR_N ? 1 : 0;
    q.splits = h->splits;
    q.c_dtype = p.c_dtype;
    q.x_dtype = p.x_dtype;
    q.d_dtype = p.d_dtype;
    q.y_dtype = p.y_dtype;
    q.int_path = int_path ? 1 : 0;
    q.alpha = alpha;
    q.beta = beta;
    q.xf = x_factor;
    q.ialpha = p.ialpha;
    q.ibeta = p.ibeta;
    q.ix = p.ix;
    q.relu = p.relu;
    const int64_t blocks = (h->tail_tiles * q.tile_m * q.tile_n / 4 + 255) / 256;
    gemm_epi::launch_splitk_epilogue(q, (int)std::min<int64_t>(blocks, (int64_t)h->cus * 8), (hipStream_t)stream);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(GEMM_EPI_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  }
  return GEMM_EPI_OK;
}

extern "C" int gemm_epi_run(const gemm_epi_handle* h, const void* A, const void* B, const void* C,
                            const void* X, void* D, void* Y, float alpha, float beta,
                            float x_factor, void* stream) {
  return run_impl(h, A, B, C, X, D, Y, alpha, beta, x_factor, stream, false);
}

extern "C" int gemm_epi_run_static(const gemm_epi_handle* h, const void* A, const void* B, const void* C,
                                   const void* X, void* D, void* Y, float alpha, float beta,
                                   float x_factor, void* stream) {
  return run_impl(h, A, B, C, X, D, Y, alpha, beta, x_factor, stream, true);
}

extern "C" int gemm_epi_destroy(gemm_epi_handle* h) {
  if (h && h->ws.load()) (void)hipFree(h->ws.load());
  delete h;
  return GEMM_EPI_OK;
}

extern "C" int gemm_epi_get_plan(const gemm_epi_handle* h, gemm_epi_plan* out) {
  if (!h || !out) return fail(GEMM_EPI_ERR_INVALID_ARG, "NULL argument");
  const Variant& v = kVariants[h->variant];
  std::memset(out, 0, sizeof *out);
  out->variant = h->variant;
  out->tile_m = v.bm;
  out->tile_n = v.bn;
  out->tile_k = v.bk;
  out->threads = v.threads;
  out->grid = h->grid;
  out->tiles = h->tiles;
  out->lds_bytes = v.lds;
  out->cus = h->cus;
  out->splits = h->splits;
  out->workspace_bytes = h->ws_bytes;
  out->split_tiles = h->splits > 1 ? h->tail_tiles : 0;
  std::snprintf(out->name, sizeof out->name, "%s", v.name);
  return GEMM_EPI_OK;
}

extern "C" int gemm_epi_variant_count(void) { return kNumVariants; }

extern "C" const char* gemm_epi_variant_name(int variant) {
  if (variant < 0 || variant >= kNumVariants) return nullptr;
  return kVariants[variant].name;
}

extern "C" const char* gemm_epi_status_string(int code) {
  switch (code) {
    case GEMM_EPI_OK: return "success";
    case GEMM_EPI_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_EPI_ERR_UNSUPPORTED: return "unsupported problem";
    case GEMM_EPI_ERR_ALIGNMENT: return "alignment requirement not met";
    case GEMM_EPI_ERR_DEVICE: return "device error";
    case GEMM_EPI_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_EPI_ERR_HOST_ALLOC: return "host allocation failed";
    default: return "unknown status";
  }
}

extern "C" const char* gemm_epi_last_error(void) { return g_last_error; }
