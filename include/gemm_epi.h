/*
 * gemm_epi.h -- C ABI of the MI355X (gfx950) fused-epilogue batched GEMM.
 *
 * The operation (CuTe DSL example "custom_epilogue_dense_gemm.py", module
 * docstring, "Tensor dimensions" and the epilogue formula it states):
 *
 *     Y[l] = A[l] . B[l]^T
 *     D[l] = alpha * (A[l] . B[l]^T) + beta * C[l] + x_factor * X[l]
 *
 * A is M x K x L, B is N x K x L, C, X, D and Y are M x N x L.  Inputs are
 * fp16, bf16, fp8 (OCP e4m3fn or e5m2), int8 or uint8; accumulation is fp32,
 * or int32 for int8 and uint8.  The epilogue runs in fp32 (int32 for int8) on the unrounded
 * accumulator and rounds to nearest-even into the output types.  By default
 * no ReLU is applied (the docstring's formula has none).  The desc field
 * `epilogue` selects instead the form the example's epilogue function builds
 * (same file, the `epilogue` function passed to the GEMM object):
 *
 *     D[l] = max(0, alpha * (A[l] . B[l]^T) + beta * C[l]) + x_factor * X[l]
 *
 * (a NaN in the clamped sum becomes 0; with int32 outputs the clamp is of the
 * wrapped int32 sum).
 *
 * Conventions (taken from the Blackwell pipeline API card, "Host side" and
 * "Device side", and the CuTe DSL example's "Constraints"):
 *   - every entry point returns a status code; gemm_epi_status_string() maps
 *     it to text and gemm_epi_last_error() gives the calling thread's detail;
 *   - everything that can be validated without the device is validated in
 *     gemm_epi_create(); nothing ever falls back silently to another path;
 *   - the contiguous extent of every tensor is a multiple of 16 bytes and
 *     every base pointer is 16-byte aligned;
 *   - C, X, D and Y share one majorness; A and B share one element type,
 *     except that the two fp8 formats may be paired (b_dtype; the pipeline
 *     API card, "Precision": fp8 e4m3 or e5m2 in any pairing);
 *   - one immutable handle per problem shape, reusable from any host thread
 *     and on any stream of the device it was created on.
 *
 * Layout: every tensor is packed, batch index outermost.  The majorness
 * letter names the contiguous mode:
 *   A  'K': A[l][m][k] at l*M*K + m*K + k     'M': at l*M*K + k*M + m
 *   B  'K': B[l][n][k] at l*N*K + n*K + k     'N': at l*N*K + k*N + n
 *   CD 'N': T[l][m][n] at l*M*N + m*N + n     'M': at l*M*N + n*M + m
 *
 * Memory ownership: all tensor pointers are device pointers owned by the
 * caller, which keeps them alive until the work queued on the stream has
 * finished.  A handle is a small host object; the only device memory the
 * library allocates is a split-K plan's workspace (see gemm_epi_run), owned
 * by the handle.
 */
#ifndef GEMM_EPI_H
#define GEMM_EPI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  GEMM_EPI_OK = 0,
  GEMM_EPI_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, bad enum */
  GEMM_EPI_ERR_UNSUPPORTED = 2, /* valid request this library does not run */
  GEMM_EPI_ERR_ALIGNMENT = 3,   /* 16-byte rule broken (extent or pointer) */
  GEMM_EPI_ERR_DEVICE = 4,      /* no usable gfx950 device / HIP query failed */
  GEMM_EPI_ERR_LAUNCH = 5,      /* the kernel launch itself failed */
  GEMM_EPI_ERR_HOST_ALLOC = 6   /* the host-side handle could not be allocated */
};

/* Element types.  GEMM_EPI_NONE marks an absent C, X or Y. */
enum {
  GEMM_EPI_NONE = 0,
  GEMM_EPI_F16 = 1,  /* IEEE binary16 */
  GEMM_EPI_BF16 = 2, /* bfloat16 */
  GEMM_EPI_E4M3 = 3, /* OCP fp8 e4m3fn (A/B only) */
  GEMM_EPI_I8 = 4,   /* int8 (A/B only) */
  GEMM_EPI_F32 = 5,  /* binary32 (C/X/D/Y only) */
  GEMM_EPI_I32 = 6,  /* int32 (C/X/D/Y only, with int8 inputs) */
  GEMM_EPI_E5M2 = 7, /* OCP fp8 e5m2 (A/B only) */
  GEMM_EPI_U8 = 8    /* uint8 (A/B only) */
};

/* Majorness: the contiguous mode of a tensor (see the table above). */
enum { GEMM_EPI_MAJOR_K = 0, GEMM_EPI_MAJOR_M = 1, GEMM_EPI_MAJOR_N = 2 };

/* Epilogue form (see the formulas above). */
enum { GEMM_EPI_LINEAR = 0, GEMM_EPI_RELU = 1 };

typedef struct gemm_epi_desc {
  int64_t M, N, K, L;  /* all >= 1 */
  int32_t a_major;     /* GEMM_EPI_MAJOR_K or _M */
  int32_t b_major;     /* GEMM_EPI_MAJOR_K or _N */
  int32_t cd_major;    /* GEMM_EPI_MAJOR_N or _M: C, X, D and Y alike */
  int32_t ab_dtype;    /* F16, BF16, E4M3, E5M2, I8 or U8 */
  int32_t c_dtype;     /* NONE, or F16/BF16/F32 (float A/B), I32 (int8/uint8 A/B) */
  int32_t x_dtype;     /* as c_dtype */
  int32_t d_dtype;     /* F16/BF16/F32 (float A/B) or I32 (int8/uint8 A/B) */
  int32_t y_dtype;     /* NONE, or as d_dtype */
  int32_t epilogue;    /* GEMM_EPI_LINEAR (0) or GEMM_EPI_RELU */
  int32_t b_dtype;     /* NONE (0): B has ab_dtype.  Else the other fp8 format
                          for an fp8 ab_dtype: E4M3 x E5M2 or E5M2 x E4M3
                          (A's format x B's) */
  int32_t splits;      /* K split: 0 = chosen by the library (when K is
                          long, the tiles of a last round that would leave
                          at least half of the compute units idle run in K
                          slices, after whole-K rounds of the other tiles;
                          with few tiles that is all of them), 1 = never,
                          n >= 2 = every tile in n slices (fewer if K has
                          fewer K tiles) */
} gemm_epi_desc;

typedef struct gemm_epi_handle gemm_epi_handle;

/* What a handle will launch (for reports and tuning). */
typedef struct gemm_epi_plan {
  int32_t variant;      /* index into the variant table */
  int32_t tile_m, tile_n, tile_k; /* workgroup tile; tile_k in elements */
  int32_t threads;      /* threads per workgroup */
  int32_t grid;         /* persistent workgroups launched */
  int64_t tiles;        /* L * ceil(M/tile_m) * ceil(N/tile_n) */
  int32_t lds_bytes;    /* LDS per workgroup */
  int32_t cus;          /* compute units of the device */
  int32_t splits;       /* K slices of a split tile (1: no split-K) */
  int64_t workspace_bytes; /* device workspace of a run (0 if none): split-K
                              partial sums (splits * split_tiles * tile_m *
                              tile_n * 4), then the uint8 sums and flipped
                              copies (see gemm_epi_run) or the fp16 copies of
                              widened fp8 operands (see gemm_epi_create) */
  int64_t split_tiles;  /* output tiles computed in K slices (0: none): the
                           last tiles of the raster, after whole-K rounds of
                           the others (all tiles when splits were asked for) */
  char name[64];        /* kernel variant name */
} gemm_epi_plan;

/* Largest split-K workspace gemm_epi_run_static can use (its static device
 * array, one per GPU). */
#define GEMM_EPI_STATIC_SCRATCH_BYTES (64LL << 20)

/*
 * Validate a problem and build an immutable plan for it.
 * Defining passages: the problem is the CuTe DSL example's module docstring
 * ("Tensor dimensions": A M x K x L with 'k' or 'm' major, B N x K x L with
 * 'n' or 'k' major, C/D/X/Y M x N x L with 'n' or 'm' major) checked against
 * its "Constraints" (supported input types, one type for A and B, one
 * majorness for C/D/X/Y, 16-byte aligned contiguous dimension); building and
 * validating the plan once, before any launch, with an error code on failure
 * is the Blackwell pipeline API card's "Host side" convention.
 * desc : problem description (read only, not retained).
 * out  : receives the new handle, or NULL on any error.
 * Static checks come first and need no device: sizes >= 1 and the packed
 * element counts within int64; dtype combinations; contiguous extents a
 * multiple of 16 bytes; one majorness for C/D/X/Y (by construction); a
 * tile's rows of A and B, and its lines of C/X/D/Y, addressable with 31-bit
 * byte offsets (GEMM_EPI_ERR_UNSUPPORTED beyond: K or the leading extent of
 * C/X/D/Y in the millions).  Then
 * the current HIP device is queried once (compute units, architecture);
 * anything but gfx950 is GEMM_EPI_ERR_DEVICE.  Allocates only the host
 * object (GEMM_EPI_ERR_HOST_ALLOC if that fails).  fp8 A/B with an fp32 D or
 * Y, and fp8 pairings and layouts without an fp8 kernel, run widened: each
 * run first converts A and B to fp16 copies in the workspace (exact: every
 * e4m3 and e5m2 value is an fp16 value; L*M*K*2 and L*N*K*2 bytes, each at
 * a 256-byte boundary, after any split-K partial sums) and an fp16 kernel
 * of the layout runs on them (so the plan names an f16 variant).  The
 * kernel is the layout's 256x256-tile variant; with desc->splits == 0 and
 * K-major A and B with N-major C/D, a smaller tile where built: 128x128
 * (fp16, bf16, e4m3, int8) when the 256x256 tiles would fill at most a
 * quarter of the compute units, 192x256 or 128x256 (fp16, bf16, e4m3,
 * int8) when the 256x256 tiles leave a partial round that those fill
 * better.  A plan of 2^31
 * or more work items (tiles and K slices) is GEMM_EPI_ERR_UNSUPPORTED.
 * Returns GEMM_EPI_OK or an error code.
 */
int gemm_epi_create(const gemm_epi_desc* desc, gemm_epi_handle** out);

/*
 * As gemm_epi_create (same passages), but forces kernel variant `variant` (0 <=
 * variant < gemm_epi_variant_count()); -1 picks the variant gemm_epi_create
 * would.  A variant that cannot run the problem is GEMM_EPI_ERR_UNSUPPORTED.
 */
int gemm_epi_create_variant(const gemm_epi_desc* desc, int variant,
                            gemm_epi_handle** out);

/*
 * Enqueue one fused GEMM on `stream` (a hipStream_t; NULL is the null
 * stream) and return without waiting.
 * Defining passages: the CuTe DSL example's epilogue function (every load of
 * C and X before any store; Y is the accumulator; D = alpha * accumulator +
 * beta * C + x_factor * X, or its clamped form) and its run() (the call goes
 * on the caller's current stream); the Blackwell pipeline API card's "Device
 * side" (one persistent grid walks every output tile with the same handle).
 * A, B, D  : required device pointers.
 * C, X     : read only; may be NULL only if their dtype is NONE or their
 *            scalar (beta, x_factor) is 0, in which case they are not read.
 * Y        : NULL exactly when y_dtype is NONE.
 * alpha, beta, x_factor : fp32 scalars.  With int32 outputs they must be
 *            integers of magnitude <= 2^24 (the epilogue is then exact int32
 *            arithmetic), else GEMM_EPI_ERR_UNSUPPORTED.
 * uint8 A/B run on the int8 MFMA: small kernels before the GEMM write copies
 * of A and B with every byte's top bit flipped (u - 128) and the sums of
 * each A row and B column of the unsigned bytes along K into the handle's
 * workspace (L*(M+N)*4 bytes of sums, then L*M*K and L*N*K bytes of copies,
 * each part at a 256-byte boundary; allocated like a split-K workspace;
 * uint8 plans never split K, and M and N must be below 2^29); every
 * accumulator starts at 128*(row sum + column sum) - 16384*K, wrapping,
 * which makes the result exact whenever it fits in int32.
 * Split-K plans (gemm_epi_plan.splits > 1) run two kernels on `stream`: the
 * K slices write fp32 (int32) partial sums to a workspace of
 * plan.workspace_bytes, then a second kernel adds them (in slice order) and
 * applies the epilogue.  Any plan with a workspace (split K, uint8, widened
 * fp8) gets it at its first run (hipMalloc; it belongs to the handle and
 * gemm_epi_destroy frees it), so runs of one such handle that overlap in
 * time on different streams race on it.
 * Every pointer must be 16-byte aligned.  D may be C itself (the same
 * pointer, with d_dtype == c_dtype): an in-place update, since each output
 * element's C is read before its D is written by the same lane.  No other
 * overlap of an output with an input or with the other output is allowed; X
 * is never written, nor C unless it is D.  Checks happen before anything is enqueued;
 * GEMM_EPI_ERR_LAUNCH reports a failed launch.  Faults inside the kernel
 * surface at the caller's next synchronisation.  Thread-safe.
 */
int gemm_epi_run(const gemm_epi_handle* h, const void* A, const void* B,
                 const void* C, const void* X, void* D, void* Y, float alpha,
                 float beta, float x_factor, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): gemm_epi_run with the
 * same arguments, checks and results, which never allocates.  A plan with a
 * workspace (split K, uint8, widened fp8) uses a file-scope device array of
 * GEMM_EPI_STATIC_SCRATCH_BYTES (one per GPU, held until the process ends)
 * as its workspace instead of the handle's; a plan whose workspace is larger
 * is GEMM_EPI_ERR_UNSUPPORTED.  Every call on one GPU shares that array
 * (everything a call reads there it wrote first in the same call, except the
 * uint8 sums of an M-major A / N-major B, which a kernel of the call zeroes
 * first, so nothing needs clearing), so calls of such plans that overlap in
 * time on one GPU race.
 */
int gemm_epi_run_static(const gemm_epi_handle* h, const void* A, const void* B,
                        const void* C, const void* X, void* D, void* Y,
                        float alpha, float beta, float x_factor, void* stream);

/* Free a handle and its split-K workspace, if any (NULL is fine).  No run on
 * it may still be being enqueued or executing.  (Tensors are the caller's:
 * the API card's "Host side" puts buffer ownership with the caller.) */
int gemm_epi_destroy(gemm_epi_handle* h);

/* Fill *out with what the handle launches (tile, grid and LDS sizes: the
 * quantities the API card's "Host side" computes for its launch). */
int gemm_epi_get_plan(const gemm_epi_handle* h, gemm_epi_plan* out);

/* Number of compiled kernel variants and the name of one. */
int gemm_epi_variant_count(void);
const char* gemm_epi_variant_name(int variant);

/* Static text for a status code ("unknown status" for anything else): the
 * error-string function of the API card's "Host side". */
const char* gemm_epi_status_string(int code);

/* Detail of the calling thread's last error ("" if none). */
const char* gemm_epi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPI_H */
