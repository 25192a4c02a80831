/*
 * gemm_epi_oracle.c -- CPU oracle for the fused-epilogue batched GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; it exists so that tests, the smoke check and the bench's
 * CPU-baseline leg can compare the GPU library against a plain, slow,
 * obviously correct definition.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes (from "custom_epilogue_dense_gemm.py", the CuTe DSL
 * Blackwell example, module docstring, "Tensor dimensions" and the fused
 * epilogue it describes):
 *
 *     Y[l,m,n] = sum_k A[l,m,k] * B[l,n,k]
 *     D[l,m,n] = alpha * Y[l,m,n] + beta * C[l,m,n] + x_factor * X[l,m,n]
 *
 * and, as an option, the form of the example's epilogue function (the code
 * that builds the epilogue in the same file), which clamps the scaled
 * accumulator plus the C term at zero before the X term is added:
 *
 *     D[l,m,n] = max(0, alpha * Y[l,m,n] + beta * C[l,m,n]) + x_factor * X[l,m,n]
 *
 * Inputs: fp16, bf16, OCP fp8 E4M3 and E5M2, int8, uint8; B may have its own type
 * (the fp8 pairs E4M3 x E5M2 and E5M2 x E4M3).  A is M x K x L, B is N x K x L (so the product is A times B-transposed in
 * row-major algebra), C/X/D/Y are M x N x L.  Every stored element is decoded
 * exactly to double, the contraction runs in double in ascending k, and the
 * epilogue is applied in double to the unrounded sum.  Nothing is rounded to
 * the output type: the caller compares the GPU's stored output against these
 * doubles with a normalised error, using the side sum S = sum_k |a|*|b|
 * that this file also returns.
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of the repository):
 *   - no ReLU by default: the module docstring's formula has none; the
 *     clamped form is the separate option above;
 *   - D is formed from the accumulator, not from the rounded Y;
 *   - a C (X) term is skipped when C (X) is absent or beta (x_factor) is 0;
 *   - batches are packed, L outermost; the majorness letter names the
 *     contiguous mode (A 'K'/'M', B 'K'/'N', C/D/X/Y 'N'/'M').
 *
 * Parity pins: every function here is checked by the CPU tests against
 * values fixed by the number formats' definitions, exact rational brute
 * force, closed forms and an independent fp64 library matmul.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Storage types understood by the oracle (its own numbering). */
enum {
  ORC_NONE = 0,
  ORC_F16 = 1,  /* IEEE 754 binary16 */
  ORC_BF16 = 2, /* bfloat16: upper half of binary32 */
  ORC_E4M3 = 3, /* OCP fp8 E4M3FN: bias 7, no infinities, S.1111.111 is NaN */
  ORC_I8 = 4,
  ORC_F32 = 5,
  ORC_I32 = 6,
  ORC_E5M2 = 7, /* OCP fp8 E5M2: bias 15, IEEE-like infinities and NaNs */
  ORC_U8 = 8    /* unsigned 8-bit integer, 0..255 */
};

typedef struct {
  int64_t M, N, K, L;
  int32_t a_mmajor;  /* 0: A[l][m][k] (k contiguous); 1: A[l][k][m] */
  int32_t b_nmajor;  /* 0: B[l][n][k] (k contiguous); 1: B[l][k][n] */
  int32_t cd_mmajor; /* 0: C/D/X/Y[l][m][n] (n contiguous); 1: [l][n][m] */
  int32_t ab_type, c_type, x_type;
  int32_t b_type; /* ORC_NONE: B has A's type; else B's own type (fp8 pairs) */
} orc_desc;

/* ---- exact decoders, written from the format definitions ---------------- */

static double dec_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f/2^10 * 2^-14 */
  else if (e == 31)
    v = (f == 0) ? INFINITY : NAN;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1+f/2^10) * 2^(e-15) */
  return s ? -v : v;
}

static double dec_bf16(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 255, f = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* f/2^7 * 2^-126 */
  else if (e == 255)
    v = (f == 0) ? INFINITY : NAN;
  else
    v = ldexp((double)(128 + f), e - 134); /* (1+f/2^7) * 2^(e-127) */
  return s ? -v : v;
}

static double dec_e4m3(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, f = b & 7;
  double v;
  if (e == 15 && f == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)f, -9); /* f/2^3 * 2^-6 */
  else
    v = ldexp((double)(8 + f), e - 10); /* (1+f/2^3) * 2^(e-7) */
  return s ? -v : v;
}

static double dec_e5m2(uint8_t b) {
  int s = b >> 7, e = (b >> 2) & 31, f = b & 3;
  double v;
  if (e == 31)
    v = (f == 0) ? INFINITY : NAN;
  else if (e == 0)
    v = ldexp((double)f, -16); /* f/2^2 * 2^-14 */
  else
    v = ldexp((double)(4 + f), e - 17); /* (1+f/2^2) * 2^(e-15) */
  return s ? -v : v;
}

static double dec_f32(uint32_t w) {
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double load(const void* p, int type, int64_t i) {
  switch (type) {
    case ORC_F16: return dec_f16(((const uint16_t*)p)[i]);
    case ORC_BF16: return dec_bf16(((const uint16_t*)p)[i]);
    case ORC_E4M3: return dec_e4m3(((const uint8_t*)p)[i]);
    case ORC_E5M2: return dec_e5m2(((const uint8_t*)p)[i]);
    case ORC_I8: return (double)((const int8_t*)p)[i];
    case ORC_U8: return (double)((const uint8_t*)p)[i];
    case ORC_F32: return dec_f32(((const uint32_t*)p)[i]);
    case ORC_I32: return (double)((const int32_t*)p)[i];
    default: return NAN;
  }
}

/* Decode n stored elements to double (exposed so tests can pin decoding). */
int orc_decode(int type, const void* src, int64_t n, double* out) {
  if (type < ORC_F16 || type > ORC_U8 || (n > 0 && (!src || !out))) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = load(src, type, i);
  return 0;
}

/* ---- element addressing (packed batches, L outermost) ------------------- */

static int64_t a_index(const orc_desc* d, int64_t l, int64_t m, int64_t k) {
  return l * d->M * d->K + (d->a_mmajor ? k * d->M + m : m * d->K + k);
}
static int64_t b_index(const orc_desc* d, int64_t l, int64_t n, int64_t k) {
  return l * d->N * d->K + (d->b_nmajor ? k * d->N + n : n * d->K + k);
}
static int64_t cd_index(const orc_desc* d, int64_t l, int64_t m, int64_t n) {
  return l * d->M * d->N + (d->cd_mmajor ? n * d->M + m : m * d->N + n);
}

/* ---- one output element: contraction then epilogue ----------------------- */

typedef struct {
  const orc_desc* d;
  const void *A, *B, *C, *X;
  double alpha, beta, xf;
  int relu; /* clamp alpha*Y + beta*C at zero before the X term */
} orc_problem;

static void element(const orc_problem* p, int64_t l, int64_t m, int64_t n,
                    double* dref, double* yref, double* sref) {
  const orc_desc* d = p->d;
  double acc = 0.0, s = 0.0;
  for (int64_t k = 0; k < d->K; ++k) {
    double a = load(p->A, d->ab_type, a_index(d, l, m, k));
    double b = load(p->B, d->b_type ? d->b_type : d->ab_type, b_index(d, l, n, k));
    acc += a * b;
    s += fabs(a) * fabs(b);
  }
  double out = p->alpha * acc;
  int64_t o = cd_index(d, l, m, n);
  if (p->C && d->c_type != ORC_NONE && p->beta != 0.0)
    out += p->beta * load(p->C, d->c_type, o);
  if (p->relu && !(out > 0.0)) out = 0.0;
  if (p->X && d->x_type != ORC_NONE && p->xf != 0.0)
    out += p->xf * load(p->X, d->x_type, o);
  if (dref) *dref = out;
  if (yref) *yref = acc;
  if (sref) *sref = s;
}

/* ---- threading: rows of work split across plain pthreads ---------------- */

typedef struct {
  const orc_problem* p;
  int64_t begin, end; /* range of work items */
  int mode;           /* 0: full (item = l*M+m row), 1: listed points */
  const int64_t* pts;
  double *dref, *yref, *sref;
} orc_job;

static void* run_job(void* arg) {
  orc_job* j = (orc_job*)arg;
  const orc_desc* d = j->p->d;
  for (int64_t it = j->begin; it < j->end; ++it) {
    if (j->mode == 0) {
      int64_t l = it / d->M, m = it % d->M;
      for (int64_t n = 0; n < d->N; ++n) {
        int64_t o = cd_index(d, l, m, n);
        element(j->p, l, m, n, j->dref ? j->dref + o : 0,
                j->yref ? j->yref + o : 0, j->sref ? j->sref + o : 0);
      }
    } else {
      const int64_t* q = j->pts + 3 * it;
      element(j->p, q[0], q[1], q[2], j->dref ? j->dref + it : 0,
              j->yref ? j->yref + it : 0, j->sref ? j->sref + it : 0);
    }
  }
  return 0;
}

static int run_threads(const orc_problem* p, int64_t items, int mode,
                       const int64_t* pts, double* dref, double* yref,
                       double* sref, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > items) nthreads = items > 0 ? (int)items : 1;
  orc_job jobs[256];
  pthread_t tid[256];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].p = p;
    jobs[t].begin = items * t / nthreads;
    jobs[t].end = items * (t + 1) / nthreads;
    jobs[t].mode = mode;
    jobs[t].pts = pts;
    jobs[t].dref = dref;
    jobs[t].yref = yref;
    jobs[t].sref = sref;
  }
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&tid[t], 0, run_job, &jobs[t]) != 0) {
      rc = 3;
      break;
    }
    started = t;
  }
  run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(tid[t], 0);
  if (rc) /* finish the ranges whose thread never started */
    for (int t = started + 1; t < nthreads; ++t) run_job(&jobs[t]);
  return 0;
}

static int check_desc(const orc_desc* d, const void* A, const void* B) {
  if (!d || !A || !B) return 1;
  if (d->M < 0 || d->N < 0 || d->K < 0 || d->L < 0) return 1;
  if ((d->ab_type < ORC_F16 || d->ab_type > ORC_I8) && d->ab_type != ORC_E5M2 && d->ab_type != ORC_U8)
    return 1;
  if (d->b_type != ORC_NONE && (d->b_type < ORC_F16 || d->b_type > ORC_I8) && d->b_type != ORC_E5M2 &&
      d->b_type != ORC_U8)
    return 1;
  return 0;
}

/* Full result, stored in the C/D layout of the descriptor.  Any of dref,
 * yref, sref may be NULL.  Returns 0 on success. */
int orc_gemm_epi_full(const orc_desc* d, const void* A, const void* B,
                      const void* C, const void* X, double alpha, double beta,
                      double xf, int relu, double* dref, double* yref,
                      double* sref, int nthreads) {
  if (check_desc(d, A, B)) return 1;
  orc_problem p = {d, A, B, C, X, alpha, beta, xf, relu != 0};
  return run_threads(&p, d->L * d->M, 0, 0, dref, yref, sref, nthreads);
}

/* Listed points: pts holds npts triples (l, m, n); outputs are per point. */
int orc_gemm_epi_points(const orc_desc* d, const void* A, const void* B,
                        const void* C, const void* X, double alpha,
                        double beta, double xf, int relu, int64_t npts,
                        const int64_t* pts, double* dref, double* yref,
                        double* sref, int nthreads) {
  if (check_desc(d, A, B) || npts < 0 || (npts && !pts)) return 1;
  for (int64_t i = 0; i < npts; ++i) {
    const int64_t* q = pts + 3 * i;
    if (q[0] < 0 || q[0] >= d->L || q[1] < 0 || q[1] >= d->M || q[2] < 0 ||
        q[2] >= d->N)
      return 2;
  }
  orc_problem p = {d, A, B, C, X, alpha, beta, xf, relu != 0};
  return run_threads(&p, npts, 1, pts, dref, yref, sref, nthreads);
}
