/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for guarded BF16
 * attention.  TEST INFRASTRUCTURE ONLY (see oracle.h): never linked into, or
 * called by, the product path.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (oracle/build_oracle.py).  No
 * contraction, no reassociation: every fp32 step below is one IEEE binary32
 * operation, every fp64 step one binary64 operation.
 *
 * Page citations use the keys of oracle.h: [R] the priors.kr review, [S] the
 * bud-325 summary.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORC_VERSION 2  /* bump with every change to a struct shared with Python */
#define U24 5.9604644775390625e-08 /* 2^-24: unit roundoff of binary32 */

int orc_version(void) { return ORC_VERSION; }

/* ======================================================================
 * BF16.  [R] "Why it matters" (paper §2.1): BF16 keeps FP32's 8 exponent
 * bits and 7 mantissa bits, so values in [1,2) are spaced 1/128.
 * [R] "Core idea", intuition (paper App. B): results are rounded to the
 * nearest representable value, and an exact half-way case goes to the value
 * whose last mantissa bit is even.
 * ====================================================================== */

/* Nearest bf16 to an fp32 value, written from the definition: the candidate
 * below in magnitude is the 16-bit truncation; the discarded low half decides
 * (more than half: away from zero; less: keep; exactly half: the even one). */
uint16_t orc_bf16_from_f32(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays NaN (quiet) */
  uint32_t sign = u & 0x80000000u;
  uint32_t mag = u & 0x7fffffffu;
  uint32_t below = mag & 0xffff0000u;
  uint32_t rest = mag & 0x0000ffffu;
  int away;
  if (rest > 0x8000u)
    away = 1;
  else if (rest < 0x8000u)
    away = 0;
  else
    away = (int)((below >> 16) & 1u); /* tie: go to the even neighbour */
  /* one step up in magnitude; a carry out of the mantissa moves to the next
   * binade, and out of the largest finite value to infinity, as RNE requires */
  uint32_t res = below + (away ? 0x10000u : 0u);
  return (uint16_t)((sign | res) >> 16);
}

float orc_f32_from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void orc_bf16_from_f32_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(x[i]);
}

void orc_f32_from_bf16_array(const uint16_t* h, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_from_bf16(h[i]);
}

/* Spacing of the bf16 grid in the binade of |x| (subnormal spacing below
 * 2^-126).  bf16 has 7 stored mantissa bits, so the spacing in [2^e, 2^e+1)
 * is 2^(e-7). */
double orc_bf16_ulp(double x) {
  double a = fabs(x);
  if (a == 0.0 || !isfinite(a)) return ldexp(1.0, -133);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int lo = e - 1;
  if (lo < -126) lo = -126;
  return ldexp(1.0, lo - 7);
}

/* Direct round-to-nearest-even of a double to bf16: scale by the grid
 * spacing (exact, a power of two), round the quotient to the nearest integer
 * with ties to even, scale back. */
uint16_t orc_bf16_from_f64(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xffc0u : 0x7fc0u);
  if (x == 0.0) return (uint16_t)(signbit(x) ? 0x8000u : 0x0000u);
  double a = fabs(x);
  uint16_t sign = (uint16_t)(signbit(x) ? 0x8000u : 0u);
  if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
  double sp = orc_bf16_ulp(a);
  double qv = a / sp;
  double rn = nearbyint(qv); /* default mode: nearest, ties to even */
  double res = rn * sp;
  if (res >= 0x1p128) return (uint16_t)(sign | 0x7f80u); /* overflow */
  float f = (float)res; /* exact: res is on the bf16 grid */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* Distance from x to the nearest rounding boundary (half-way point between
 * two neighbouring bf16 values).  A value whose error bound is smaller than
 * this rounds the same way whatever the error is. */
double orc_bf16_boundary_distance(double x) {
  double a = fabs(x);
  if (!isfinite(a)) return 0.0;
  double sp = orc_bf16_ulp(a);
  double qv = a / sp;
  double fr = qv - floor(qv);
  return fabs(fr - 0.5) * sp;
}

/* ======================================================================
 * FP8 E4M3 in the OCP 8-bit floating-point format: 1 sign bit, 4 exponent
 * bits (bias 7), 3 mantissa bits; normals from 2^-6 to 448 = 1.75 * 2^8,
 * subnormals k * 2^-9, no infinities (the all-ones pattern is NaN).
 * Rounding: to nearest, ties to even; magnitudes that round past 448 are
 * NaN here (the variant never produces them).
 * ====================================================================== */
double orc_e4m3_ulp(double x) {
  double a = fabs(x);
  if (a == 0.0 || !isfinite(a)) return ldexp(1.0, -9);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int lo = e - 1;
  if (lo < -6) lo = -6;
  return ldexp(1.0, lo - 3);
}

double orc_e4m3_round(double x) {
  if (isnan(x) || x == 0.0) return x;
  double a = fabs(x);
  if (isinf(a)) return NAN;
  double sp = orc_e4m3_ulp(a);
  double res = nearbyint(a / sp) * sp; /* default mode: nearest, ties to even */
  if (res > 448.0) return NAN;
  return signbit(x) ? -res : res;
}

double orc_e4m3_boundary_distance(double x) {
  double a = fabs(x);
  if (!isfinite(a)) return 0.0;
  double sp = orc_e4m3_ulp(a);
  double qv = a / sp;
  double fr = qv - floor(qv);
  return fabs(fr - 0.5) * sp;
}

/* ======================================================================
 * FP4 E2M1 (OCP MX element format): sign, 2 exponent bits (bias 1), 1
 * mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or
 * NaN.  MX scaling: a block of values shares the scale X = 2^(floor(log2
 * amax) - 2) (E8M0; 2 is the element format's largest exponent) and each
 * element is RNE(clamp(v / X, -6, 6)) on the E2M1 grid.
 * ====================================================================== */
double orc_e2m1_round(double y) {
  double a = fabs(y);
  if (isnan(y)) return y;
  if (a > 6.0) a = 6.0; /* saturate */
  double sp = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
  double r = nearbyint(a / sp) * sp; /* ties to even: to the even multiple */
  /* at a binade edge the even neighbour is the larger one (2, 4) */
  if (r > 6.0) r = 6.0;
  return signbit(y) ? -r : r;
}

double orc_e2m1_spacing(double y) {
  double a = fabs(y);
  return a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
}

/* Distance of y to the nearest E2M1 rounding midpoint (0.25, 0.75, 1.25,
 * 1.75, 2.5, 3.5 or 5; beyond 5 everything rounds to 6). */
double orc_e2m1_boundary_distance(double y) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  double a = fabs(y), d = INFINITY;
  for (int i = 0; i < 7; ++i) d = fmin(d, fabs(a - mid[i]));
  return d;
}

/* Exponent of the MX scale of a block with largest magnitude amax:
 * floor(log2 amax) - 2, as the E8M0 byte (bias 127), at least 1. */
int orc_mx_scale_byte(double amax) {
  if (!(amax > 0.0)) return 1;
  int e;
  frexp(amax, &e); /* amax in [2^(e-1), 2^e) */
  int b = 127 + (e - 1) - 2;
  return b < 1 ? 1 : (b > 254 ? 254 : b);
}

/* The same with ceil(log2 amax): one more unless amax is a power of two. */
int orc_mx_scale_byte_ceil(double amax) {
  if (!(amax > 0.0)) return 1;
  int e;
  double f = frexp(amax, &e); /* f in [0.5, 1) */
  int b = 127 + (e - 1) - 2 + (f != 0.5 ? 1 : 0);
  return b < 1 ? 1 : (b > 254 ? 254 : b);
}

/* Error-free transformation of a + b (Knuth's TwoSum). */
static void two_sum(double a, double b, double* s, double* e) {
  double x = a + b;
  double bv = x - a;
  double av = x - bv;
  *s = x;
  *e = (a - av) + (b - bv);
}

/* Sum kept as an unevaluated pair hi + lo (twice double precision). */
typedef struct {
  double hi, lo;
} dd_t;

static void dd_add(dd_t* acc, double x) {
  double s, e;
  two_sum(acc->hi, x, &s, &e);
  double lo = acc->lo + e;
  two_sum(s, lo, &acc->hi, &acc->lo);
}

/* RNE to bf16 of hi + lo.  |lo| is below half a double ulp of hi, so it can
 * only matter when hi sits exactly on a bf16 half-way point. */
static uint16_t dd_to_bf16(dd_t v) {
  if (v.lo != 0.0 && orc_bf16_boundary_distance(v.hi) == 0.0 && isfinite(v.hi)) {
    double sp = orc_bf16_ulp(v.hi);
    double toward = (v.lo > 0.0) ? v.hi + sp / 4 : v.hi - sp / 4;
    return orc_bf16_from_f64(toward);
  }
  return orc_bf16_from_f64(v.hi);
}

/* [R] "Core idea", equations (paper §3.3.2) and [S] "Results": the
 * unnormalised output is accumulated wider than bf16 and rounded once; the
 * small same-sign residual survives in the accumulator and decides a
 * half-way case.  This is that step: RNE of the exact sum. */
uint16_t orc_bf16_round_of_sum(const double* terms, int32_t n, double* exact_out) {
  dd_t acc = {0.0, 0.0};
  for (int32_t i = 0; i < n; ++i) dd_add(&acc, terms[i]);
  if (exact_out) *exact_out = acc.hi + acc.lo;
  return dd_to_bf16(acc);
}

/* ======================================================================
 * Shared plumbing: problem checks, head lists, a tiny thread pool.
 * ====================================================================== */

static int check_problem(const orc_problem* p) {
  if (!p) return -1;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seqlen <= 0 ||
      p->head_dim <= 0)
    return -2;
  if (p->heads_q % p->heads_kv != 0) return -2;
  if (p->guard < ORC_GUARD_NONE || p->guard > ORC_GUARD_EPS) return -4;
  if (!(p->alpha > 0.0f)) return -4;
  return 0;
}

/* A head list (NULL: every head) names only heads of the problem: each index
 * in [0, count), count = batch * heads. */
static int heads_valid(const int32_t* heads, int32_t n, int32_t count) {
  if (!heads) return 1;
  if (n < 0) return 0;
  for (int32_t i = 0; i < n; ++i)
    if (heads[i] < 0 || heads[i] >= count) return 0;
  return 1;
}

typedef struct {
  void (*fn)(void* ctx, int32_t item);
  void* ctx;
  int32_t nitems;
  int32_t nthreads;
  int32_t tid;
} pool_arg;

static void* pool_worker(void* a) {
  pool_arg* pa = (pool_arg*)a;
  for (int32_t i = pa->tid; i < pa->nitems; i += pa->nthreads) pa->fn(pa->ctx, i);
  return NULL;
}

/* Run fn(ctx, i) for i in [0, nitems) on nthreads threads (static split). */
static void run_pool(void (*fn)(void*, int32_t), void* ctx, int32_t nitems, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nitems) nthreads = nitems;
  if (nthreads <= 1) {
    for (int32_t i = 0; i < nitems; ++i) fn(ctx, i);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  pool_arg* args = (pool_arg*)malloc(sizeof(pool_arg) * (size_t)nthreads);
  for (int32_t t = 0; t < nthreads; ++t) {
    args[t].fn = fn;
    args[t].ctx = ctx;
    args[t].nitems = nitems;
    args[t].nthreads = nthreads;
    args[t].tid = t;
    pthread_create(&th[t], NULL, pool_worker, &args[t]);
  }
  for (int32_t t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(args);
}

/* Work items over (listed head, block of rows).  Rows of a head are
 * independent in the forward functions below, so a call with few heads (a
 * single full-size head, say) splits each head into blocks of rows to keep
 * every thread busy; each row's arithmetic is the same either way. */
typedef struct {
  int32_t nblk, rows; /* blocks per head, rows per block */
} row_split;

static row_split split_rows(int32_t nheads, int32_t N, int32_t nthreads) {
  row_split r = {1, N};
  if (nthreads > 1 && nheads > 0 && nheads < 4 * nthreads) {
    int32_t want = (8 * nthreads + nheads - 1) / nheads;
    if (want > N) want = N;
    r.rows = (N + want - 1) / want;
    r.nblk = (N + r.rows - 1) / r.rows;
  }
  return r;
}

/* Head and row range of work item `item`. */
static void split_item(row_split r, int32_t item, const int32_t* heads, int32_t N,
                       int32_t* qh, int32_t* i_begin, int32_t* i_end) {
  int32_t h = item / r.nblk, b = item % r.nblk;
  *qh = heads ? heads[h] : h;
  *i_begin = b * r.rows;
  *i_end = *i_begin + r.rows < N ? *i_begin + r.rows : N;
}

/* Pointers to the [N][d] slabs of query head (b, h) and of its KV head.
 * Grouped-query mapping: query head h reads KV head h / (heads_q/heads_kv). */
static size_t q_head_offset(const orc_problem* p, int32_t qhead) {
  return (size_t)qhead * (size_t)p->seqlen * (size_t)p->head_dim;
}
static size_t kv_head_offset(const orc_problem* p, int32_t qhead) {
  int32_t b = qhead / p->heads_q, h = qhead % p->heads_q;
  int32_t g = p->heads_q / p->heads_kv;
  int32_t hk = h / g;
  return ((size_t)b * (size_t)p->heads_kv + (size_t)hk) * (size_t)p->seqlen * (size_t)p->head_dim;
}

/* Keys visible to query row i. */
static int32_t visible(const orc_problem* p, int32_t i) {
  return p->causal ? i + 1 : p->seqlen;
}

/* s = sum_f q_f k_f in double: each product of two bf16 values is exact in
 * double and the sum of head_dim of them stays exact for these magnitudes. */
static double dot_bf16(const uint16_t* a, const uint16_t* b, int32_t d) {
  double s = 0.0;
  for (int32_t f = 0; f < d; ++f)
    s += (double)orc_f32_from_bf16(a[f]) * (double)orc_f32_from_bf16(b[f]);
  return s;
}

/* Error bound of a sum c0 + sum(terms) as the kernel computes it (see
 * orc_schedule).  With chunk = 0: any order of fp32 additions.  Otherwise a
 * chain of matrix instructions, each adding `chunk` products to the running
 * value C.  Bound of one instruction (bf16 inputs, fp32 accumulate), from
 * measurements of the hardware (no simple model reproduces its outputs bit
 * for bit; this bound covers every measured one): with E the exponent of the
 * largest magnitude among the chunk's products and C, the result differs
 * from the exact sum by less than 2^(E-24) for every product that is not a
 * multiple of 2^(E-24), another 2^(E-24) for C, u*sum|p| for partial sums
 * rounded to fp32 and 4u*|result| (two units in the result's last place:
 * measured where the sum leaves C's binade) for the final rounding (u =
 * 2^-24).  chunk_err scales the whole bound (a safety factor over the
 * measured worst case).                                                   */
static double chain_bound(const orc_schedule* sc, double c0, const double* terms, int32_t n) {
  if (!sc || sc->chunk <= 0) {
    double a = fabs(c0);
    for (int32_t i = 0; i < n; ++i) a += fabs(terms[i]);
    return (double)(n + 1) * U24 * a;
  }
  double err = 0.0, c = c0;
  double factor = sc->chunk_err > 0 ? sc->chunk_err : 1.0;
  for (int32_t i0 = 0; i0 < n; i0 += sc->chunk) {
    int32_t i1 = i0 + sc->chunk < n ? i0 + sc->chunk : n;
    double sa = 0.0, r = c, mx = fabs(c);
    for (int32_t i = i0; i < i1; ++i) {
      sa += fabs(terms[i]);
      r += terms[i];
      if (fabs(terms[i]) > mx) mx = fabs(terms[i]);
    }
    double step = 0.0;
    if (mx > 0.0) {
      int e;
      frexp(mx, &e); /* mx in [2^(e-1), 2^e) */
      double grid = ldexp(1.0, (e - 1) - 24);
      for (int32_t i = i0; i < i1; ++i) {
        double qv = terms[i] / grid; /* exact: grid is a power of two */
        if (qv != floor(qv)) step += grid;
      }
      if (c != 0.0) step += grid;
      step += U24 * sa;
    }
    step += 4.0 * U24 * fabs(r); /* up to two units in the result's last place */
    err += factor * step;
    c = r;
  }
  return err;
}

/* E4M3 exponent of a nonzero value: floor(log2|x|) for normals, -6 for the
 * subnormals (the format's smallest normal exponent). */
static int e4m3_exponent(double x) {
  int e;
  frexp(fabs(x), &e); /* |x| in [2^(e-1), 2^e) */
  return e - 1 < -6 ? -6 : e - 1;
}

/* Error bound of c0 + sum(terms) where the terms are products a*b of E4M3
 * operands (pv_fp8), esum[i] = e4m3_exponent(a) + e4m3_exponent(b), summed by
 * a chain of FP8 matrix instructions of `chunk` products each.  Model of one
 * instruction, taken from measurements of the hardware (not from the pages):
 * the products are summed in two halves; each half's products are aligned to
 * the half's largest exponent sum E and cut toward zero below 2^(E-13); the
 * accumulator input is cut below 2^(Emax-24) (Emax over both halves); the
 * total is rounded to fp32 once.  The bound does not need the halves: with
 * Emax over the instruction, a product off the grid 2^(Emax-13) loses less
 * than 2^(Emax-13) and one on it loses nothing; C loses less than
 * 2^(Emax-24) unless it is on that grid; the rounding costs u*|result|.  The
 * measured worst case reached 0.99 of this bound; it is doubled here, and
 * chunk_err scales it further.  `shift` converts exponent sums to the units
 * of the terms (terms = products * 2^shift).
 * The scaled 64-product instruction (pv_chunk = 64), also measured: its
 * products are summed in eight groups of eight, each aligned to its own
 * largest exponent sum and cut below 2^(E-13), and the group sums are cut
 * below 2^(Emax-24) when they are combined, so each group adds up to
 * 2^(Emax-24) more; with that term the bound held on every one of 786k
 * probed outputs (worst 0.98 of it), before the doubling.                 */
static double chain_bound_fp8(const orc_schedule* sc, double c0, const double* terms,
                              const int* esum, int32_t n, int shift) {
  double err = 0.0, c = c0;
  double factor = 2.0 * (sc->chunk_err > 0 ? sc->chunk_err : 1.0);
  int32_t chunk = sc->pv_chunk > 0 ? sc->pv_chunk : 16;
  const int groups = chunk > 16 ? chunk / 8 : 0; /* the group-sum term */
  for (int32_t i0 = 0; i0 < n; i0 += chunk) {
    int32_t i1 = i0 + chunk < n ? i0 + chunk : n;
    double r = c, step = 0.0;
    int emax = INT32_MIN;
    for (int32_t i = i0; i < i1; ++i) {
      r += terms[i];
      if (terms[i] != 0.0 && esum[i] > emax) emax = esum[i];
    }
    if (emax != INT32_MIN) {
      double grid = ldexp(1.0, emax - 13 + shift);
      for (int32_t i = i0; i < i1; ++i) {
        double qv = terms[i] / grid; /* exact: grid is a power of two */
        if (qv != floor(qv)) step += grid;
      }
      double gc = ldexp(1.0, emax - 24 + shift);
      if (c / gc != floor(c / gc)) step += gc;
      step += groups * gc;
    }
    step += U24 * fabs(r);
    err += factor * step;
    c = r;
  }
  return err;
}

/* Error bound of c0 + sum(terms) on the scaled FP4 matrix instruction
 * (pv_mxfp4): one instruction per `n` terms (the 64 keys of a step).  Model
 * measured on the hardware (not from the pages): the total differs from the
 * exact sum rounded to fp32 by less than 2^(Ep-24) per nonzero product (Ep
 * the exponent of the largest product) plus 2^(Epc-24) (Epc the exponent of
 * the larger of that product and |C|); this held on every measured output
 * with 0.67 of it to spare.  Doubled here; chunk_err scales it further.   */
static double chain_bound_mx(const orc_schedule* sc, double c0, const double* terms, int32_t n) {
  double factor = 2.0 * (sc->chunk_err > 0 ? sc->chunk_err : 1.0);
  double r = c0, pm = 0.0;
  int nz = 0;
  for (int32_t i = 0; i < n; ++i) {
    r += terms[i];
    if (terms[i] != 0.0) ++nz;
    pm = fmax(pm, fabs(terms[i]));
  }
  double step = 2.0 * U24 * fabs(r);
  if (pm > 0.0) {
    int ep, epc;
    frexp(pm, &ep);
    frexp(fmax(pm, fabs(c0)), &epc);
    step += nz * ldexp(1.0, ep - 1 - 24) + ldexp(1.0, epc - 1 - 24);
  }
  return factor * step;
}

/* The three bounds above, callable on their own (their CPU tests check them
 * against independent simulations of the instruction models). */
double orc_chain_bound(const orc_schedule* sc, double c0, const double* terms, int32_t n) {
  return chain_bound(sc, c0, terms, n);
}
double orc_chain_bound_fp8(const orc_schedule* sc, double c0, const double* terms,
                           const int32_t* esum, int32_t n, int32_t shift) {
  return chain_bound_fp8(sc, c0, terms, esum, n, shift);
}
double orc_chain_bound_mx(const orc_schedule* sc, double c0, const double* terms, int32_t n) {
  return chain_bound_mx(sc, c0, terms, n);
}

/* Exact score and the bound on the kernel's fp32 score for one (i, j). */
static double dot_with_bound(const orc_schedule* sc, const uint16_t* a, const uint16_t* b,
                             int32_t d, double* tmp, double* bound) {
  double s = 0.0;
  for (int32_t f = 0; f < d; ++f) {
    tmp[f] = (double)orc_f32_from_bf16(a[f]) * (double)orc_f32_from_bf16(b[f]);
    s += tmp[f];
  }
  *bound = chain_bound(sc, 0.0, tmp, d);
  return s;
}

/* ======================================================================
 * FP64 reference forward: O = softmax(alpha * Q K^T) V.
 * [R] "Core idea", equations: S = QK^T with P = softmax and O = PV; the
 * score scale alpha = 1/sqrt(d) ([S] "Method", Eqn. 2's 1/sqrt(d)).
 * ====================================================================== */

typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v;
  const int32_t* heads;
  double *o, *lse;
  row_split rs;
} fwd64_ctx;

static void fwd64_head(void* c, int32_t item) {
  fwd64_ctx* x = (fwd64_ctx*)c;
  const orc_problem* p = x->p;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t qh, i_begin, i_end;
  split_item(x->rs, item, x->heads, N, &qh, &i_begin, &i_end);
  const uint16_t* Q = x->q + q_head_offset(p, qh);
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  const uint16_t* V = x->v + kv_head_offset(p, qh);
  double* t = (double*)malloc(sizeof(double) * (size_t)N);
  double alpha = (double)p->alpha;
  for (int32_t i = i_begin; i < i_end; ++i) {
    int32_t n = visible(p, i);
    double mx = -INFINITY;
    for (int32_t j = 0; j < n; ++j) {
      t[j] = alpha * dot_bf16(Q + (size_t)i * d, K + (size_t)j * d, d);
      if (t[j] > mx) mx = t[j];
    }
    double z = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      t[j] = exp(t[j] - mx); /* now the unnormalised probability */
      z += t[j];
    }
    double* orow = x->o ? x->o + q_head_offset(p, qh) + (size_t)i * d : NULL;
    if (orow) {
      /* orow[f] = sum_j t[j] V[j][f], each sum in key order j = 0, 1, ...
       * (the loop runs over V's rows so that it reads them in memory order) */
      for (int32_t f = 0; f < d; ++f) orow[f] = 0.0;
      for (int32_t j = 0; j < n; ++j)
        for (int32_t f = 0; f < d; ++f) orow[f] += t[j] * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
      for (int32_t f = 0; f < d; ++f) orow[f] /= z;
    }
    if (x->lse) x->lse[(size_t)qh * N + i] = mx + log(z);
  }
  free(t);
}

int orc_fwd_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const int32_t* heads, int32_t nheads,
                double* o, double* lse, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v) return -1;
  if (!heads_valid(heads, nheads, p->batch * p->heads_q)) return -2;
  int32_t n = heads ? nheads : p->batch * p->heads_q;
  fwd64_ctx c = {p, q, k, v, heads, o, lse, split_rows(n, p->seqlen, nthreads)};
  run_pool(fwd64_head, &c, n * c.rs.nblk, nthreads);
  return 0;
}

/* ======================================================================
 * FP64 reference backward.
 * [R] "Core idea", equations (paper Eq. 1-2): dS = alpha P∘(dP - delta),
 * dQ = dS K, with delta = rowsum(dO∘O) ([R] summary and "method", paper §3.2).
 * dP = dO V^T, dK = dS^T Q, dV = P^T dO complete the gradient of O = PV.
 * Here dS is kept without alpha and alpha is applied in dQ and dK, which is
 * the same product.
 * ====================================================================== */

typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v, *dout;
  const int32_t* kv_heads;
  double *o, *delta, *dq, *dk, *dv;
  const double* o_in; /* nullable: the O that delta is computed from       */
  int round_ops;      /* 1: P and dS rounded to bf16 as matrix operands      */
} bwd64_ctx;

/* bf16 value of x (RNE), as a double: the matrix-operand rounding. */
static double bf16_round_d(double x) { return (double)orc_f32_from_bf16(orc_bf16_from_f64(x)); }

static void bwd64_kvhead(void* c, int32_t item) {
  bwd64_ctx* x = (bwd64_ctx*)c;
  const orc_problem* p = x->p;
  int32_t kvh = x->kv_heads ? x->kv_heads[item] : item;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t g = p->heads_q / p->heads_kv;
  int32_t b = kvh / p->heads_kv, hk = kvh % p->heads_kv;
  size_t kvoff = (size_t)kvh * (size_t)N * (size_t)d;
  const uint16_t* K = x->k + kvoff;
  const uint16_t* V = x->v + kvoff;
  double* dK = x->dk ? x->dk + kvoff : NULL;
  double* dV = x->dv ? x->dv + kvoff : NULL;
  if (dK) memset(dK, 0, sizeof(double) * (size_t)N * d);
  if (dV) memset(dV, 0, sizeof(double) * (size_t)N * d);
  double* P = (double*)malloc(sizeof(double) * (size_t)N);
  double* orow = (double*)malloc(sizeof(double) * (size_t)d);
  double* dqrow = (double*)malloc(sizeof(double) * (size_t)d);
  double* dorow = (double*)malloc(sizeof(double) * (size_t)d);
  double alpha = (double)p->alpha;
  for (int32_t hh = 0; hh < g; ++hh) {
    int32_t qh = b * p->heads_q + hk * g + hh;
    const uint16_t* Q = x->q + q_head_offset(p, qh);
    const uint16_t* dO = x->dout + q_head_offset(p, qh);
    for (int32_t i = 0; i < N; ++i) {
      int32_t n = visible(p, i);
      const uint16_t* qi = Q + (size_t)i * d;
      double mx = -INFINITY;
      for (int32_t j = 0; j < n; ++j) {
        P[j] = alpha * dot_bf16(qi, K + (size_t)j * d, d);
        if (P[j] > mx) mx = P[j];
      }
      double z = 0.0;
      for (int32_t j = 0; j < n; ++j) {
        P[j] = exp(P[j] - mx);
        z += P[j];
      }
      for (int32_t j = 0; j < n; ++j) P[j] /= z;
      /* orow[f] = sum_j P[j] V[j][f] in key order, read row by row */
      for (int32_t f = 0; f < d; ++f) {
        orow[f] = 0.0;
        dorow[f] = (double)orc_f32_from_bf16(dO[(size_t)i * d + f]);
      }
      for (int32_t j = 0; j < n; ++j)
        for (int32_t f = 0; f < d; ++f) orow[f] += P[j] * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
      size_t rbase = q_head_offset(p, qh) + (size_t)i * d;
      const double* odelta = x->o_in ? x->o_in + rbase : orow;
      double delta = 0.0;
      for (int32_t f = 0; f < d; ++f) delta += dorow[f] * odelta[f];
      memset(dqrow, 0, sizeof(double) * (size_t)d);
      for (int32_t j = 0; j < n; ++j) {
        const uint16_t* kj = K + (size_t)j * d;
        const uint16_t* vj = V + (size_t)j * d;
        double dp = 0.0;
        for (int32_t f = 0; f < d; ++f) dp += dorow[f] * (double)orc_f32_from_bf16(vj[f]);
        double ds = P[j] * (dp - delta);
        double pj = P[j];
        if (x->round_ops) {
          ds = bf16_round_d(ds);
          pj = bf16_round_d(pj);
        }
        for (int32_t f = 0; f < d; ++f) dqrow[f] += alpha * ds * (double)orc_f32_from_bf16(kj[f]);
        if (dK)
          for (int32_t f = 0; f < d; ++f)
            dK[(size_t)j * d + f] += alpha * ds * (double)orc_f32_from_bf16(qi[f]);
        if (dV)
          for (int32_t f = 0; f < d; ++f) dV[(size_t)j * d + f] += pj * dorow[f];
      }
      size_t ro = q_head_offset(p, qh) + (size_t)i * d;
      if (x->round_ops) /* dQ leaves in bf16 */
        for (int32_t f = 0; f < d; ++f) dqrow[f] = bf16_round_d(dqrow[f]);
      if (x->o) memcpy(x->o + ro, orow, sizeof(double) * (size_t)d);
      if (x->dq) memcpy(x->dq + ro, dqrow, sizeof(double) * (size_t)d);
      if (x->delta) x->delta[(size_t)qh * N + i] = delta;
    }
  }
  if (x->round_ops) /* dK and dV leave in bf16 */
    for (size_t e = 0; e < (size_t)N * d; ++e) {
      if (dK) dK[e] = bf16_round_d(dK[e]);
      if (dV) dV[e] = bf16_round_d(dV[e]);
    }
  free(P);
  free(orow);
  free(dqrow);
  free(dorow);
}

int orc_bwd_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const uint16_t* dout, const int32_t* kv_heads,
                int32_t nkv, double* o, double* delta, double* dq, double* dk,
                double* dv, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout) return -1;
  if (!heads_valid(kv_heads, nkv, p->batch * p->heads_kv)) return -2;
  bwd64_ctx c = {p, q, k, v, dout, kv_heads, o, delta, dq, dk, dv, NULL, 0};
  int32_t n = kv_heads ? nkv : p->batch * p->heads_kv;
  run_pool(bwd64_kvhead, &c, n, nthreads);
  return 0;
}

/* The same backward replayed at the method's rounding points: delta from a
 * given O (the bf16 output of the forward), and P (for dV) and dS (for dK,
 * dQ) rounded to bf16 as the operands of the products; everything else in
 * double.  Used to measure the method's own error against the definition. */
int orc_bwd_emu(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const uint16_t* dout, const int32_t* kv_heads,
                int32_t nkv, const double* o_in, int32_t round_ops, double* delta,
                double* dq, double* dk, double* dv, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout) return -1;
  if (!heads_valid(kv_heads, nkv, p->batch * p->heads_kv)) return -2;
  bwd64_ctx c = {p, q, k, v, dout, kv_heads, NULL, delta, dq, dk, dv, o_in, round_ops};
  int32_t n = kv_heads ? nkv : p->batch * p->heads_kv;
  run_pool(bwd64_kvhead, &c, n, nthreads);
  return 0;
}

/* The same backward for the keys of one KV head, in two passes that can run
 * in parallel: first every query row of the group's heads (its softmax
 * maximum and normaliser, and delta), then every block of keys (dV_j =
 * sum_i P_ij dO_i and dK_j = alpha sum_i dS_ij Q_i over the rows i that see
 * key j).  The arithmetic per (i, j) is that of bwd64_kvhead above: P
 * exact, dS = P (dP - delta), and with round_ops the bf16 operand and
 * output roundings. */
typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v, *dout;
  int32_t kvh, g;
  const double* o_in; /* nullable: [g, N, d] O rows that delta is computed from */
  int round_ops;
  double *mx, *z, *delta; /* [g, N] */
  double *dk, *dv;        /* [N, d] */
} kvkeys_ctx;

static void kvkeys_row(void* c, int32_t item) {
  kvkeys_ctx* x = (kvkeys_ctx*)c;
  const orc_problem* p = x->p;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t hh = item / N, i = item % N;
  int32_t b = x->kvh / p->heads_kv, hk = x->kvh % p->heads_kv;
  int32_t qh = b * p->heads_q + hk * x->g + hh;
  const uint16_t* qi = x->q + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* doi = x->dout + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* K = x->k + (size_t)x->kvh * N * d;
  const uint16_t* V = x->v + (size_t)x->kvh * N * d;
  double alpha = (double)p->alpha;
  int32_t n = visible(p, i);
  double* P = (double*)malloc(sizeof(double) * (size_t)n);
  double mx = -INFINITY;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = alpha * dot_bf16(qi, K + (size_t)j * d, d);
    if (P[j] > mx) mx = P[j];
  }
  double z = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = exp(P[j] - mx);
    z += P[j];
  }
  double delta = 0.0;
  for (int32_t f = 0; f < d; ++f) {
    double of;
    if (x->o_in) {
      of = x->o_in[((size_t)hh * N + i) * d + f];
    } else {
      of = 0.0;
      for (int32_t j = 0; j < n; ++j) of += (P[j] / z) * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
    }
    delta += (double)orc_f32_from_bf16(doi[f]) * of;
  }
  x->mx[item] = mx;
  x->z[item] = z;
  x->delta[item] = delta;
  free(P);
}

#define KVKEYS_BLOCK 32
static void kvkeys_block(void* c, int32_t item) {
  kvkeys_ctx* x = (kvkeys_ctx*)c;
  const orc_problem* p = x->p;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t b = x->kvh / p->heads_kv, hk = x->kvh % p->heads_kv;
  const uint16_t* K = x->k + (size_t)x->kvh * N * d;
  const uint16_t* V = x->v + (size_t)x->kvh * N * d;
  double alpha = (double)p->alpha;
  int32_t j0 = item * KVKEYS_BLOCK, j1 = j0 + KVKEYS_BLOCK < N ? j0 + KVKEYS_BLOCK : N;
  for (int32_t j = j0; j < j1; ++j) {
    double* dK = x->dk + (size_t)j * d;
    double* dV = x->dv + (size_t)j * d;
    for (int32_t f = 0; f < d; ++f) dK[f] = dV[f] = 0.0;
    const uint16_t* kj = K + (size_t)j * d;
    const uint16_t* vj = V + (size_t)j * d;
    for (int32_t hh = 0; hh < x->g; ++hh) {
      int32_t qh = b * p->heads_q + hk * x->g + hh;
      const uint16_t* Q = x->q + q_head_offset(p, qh);
      const uint16_t* dO = x->dout + q_head_offset(p, qh);
      for (int32_t i = 0; i < N; ++i) {
        if (j >= visible(p, i)) continue;
        size_t r = (size_t)hh * N + i;
        const uint16_t* qi = Q + (size_t)i * d;
        const uint16_t* doi = dO + (size_t)i * d;
        double pij = exp(alpha * dot_bf16(qi, kj, d) - x->mx[r]) / x->z[r];
        double dp = 0.0;
        for (int32_t f = 0; f < d; ++f) dp += (double)orc_f32_from_bf16(doi[f]) * (double)orc_f32_from_bf16(vj[f]);
        double ds = pij * (dp - x->delta[r]);
        if (x->round_ops) {
          ds = bf16_round_d(ds);
          pij = bf16_round_d(pij);
        }
        for (int32_t f = 0; f < d; ++f) {
          dK[f] += alpha * ds * (double)orc_f32_from_bf16(qi[f]);
          dV[f] += pij * (double)orc_f32_from_bf16(doi[f]);
        }
      }
    }
    if (x->round_ops)
      for (int32_t f = 0; f < d; ++f) {
        dK[f] = bf16_round_d(dK[f]);
        dV[f] = bf16_round_d(dV[f]);
      }
  }
}

int orc_bwd_kv_keys(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const uint16_t* dout, int32_t kv_head,
                    const double* o_in, int32_t round_ops, double* delta, double* dk,
                    double* dv, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !delta || !dk || !dv) return -1;
  if (kv_head < 0 || kv_head >= p->batch * p->heads_kv) return -2;
  int32_t N = p->seqlen, g = p->heads_q / p->heads_kv;
  double* mx = (double*)malloc(sizeof(double) * (size_t)g * N);
  double* z = (double*)malloc(sizeof(double) * (size_t)g * N);
  if (!mx || !z) {
    free(mx);
    free(z);
    return -3;
  }
  kvkeys_ctx c = {p, q, k, v, dout, kv_head, g, o_in, round_ops, mx, z, delta, dk, dv};
  run_pool(kvkeys_row, &c, g * N, nthreads);
  run_pool(kvkeys_block, &c, (N + KVKEYS_BLOCK - 1) / KVKEYS_BLOCK, nthreads);
  free(mx);
  free(z);
  return 0;
}

typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v, *dout;
  const int32_t *qheads, *rows;
  double *o, *delta, *dq;
  const double* o_in; /* nullable: [n, d] O rows that delta is computed from */
  int round_ops;      /* 1: dS rounded to bf16 as the dQ operand            */
} bwdrow_ctx;

/* One query row of the backward above, written out the same way. */
static void bwdrow_item(void* c, int32_t item) {
  bwdrow_ctx* x = (bwdrow_ctx*)c;
  const orc_problem* p = x->p;
  int32_t qh = x->qheads[item], i = x->rows[item];
  int32_t d = p->head_dim;
  const uint16_t* qi = x->q + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* doi = x->dout + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  const uint16_t* V = x->v + kv_head_offset(p, qh);
  double alpha = (double)p->alpha;
  int32_t n = visible(p, i);
  double* P = (double*)malloc(sizeof(double) * (size_t)n);
  double mx = -INFINITY;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = alpha * dot_bf16(qi, K + (size_t)j * d, d);
    if (P[j] > mx) mx = P[j];
  }
  double z = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = exp(P[j] - mx);
    z += P[j];
  }
  for (int32_t j = 0; j < n; ++j) P[j] /= z;
  double* orow = x->o + (size_t)item * d;
  double* dqrow = x->dq + (size_t)item * d;
  /* orow[f] = sum_j P[j] V[j][f] in key order, read row by row */
  for (int32_t f = 0; f < d; ++f) {
    orow[f] = 0.0;
    dqrow[f] = 0.0;
  }
  for (int32_t j = 0; j < n; ++j)
    for (int32_t f = 0; f < d; ++f) orow[f] += P[j] * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
  const double* odelta = x->o_in ? x->o_in + (size_t)item * d : orow;
  double delta = 0.0;
  for (int32_t f = 0; f < d; ++f) delta += (double)orc_f32_from_bf16(doi[f]) * odelta[f];
  for (int32_t j = 0; j < n; ++j) {
    double dp = 0.0;
    for (int32_t f = 0; f < d; ++f)
      dp += (double)orc_f32_from_bf16(doi[f]) * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
    double ds = P[j] * (dp - delta);
    if (x->round_ops) ds = bf16_round_d(ds);
    for (int32_t f = 0; f < d; ++f) dqrow[f] += alpha * ds * (double)orc_f32_from_bf16(K[(size_t)j * d + f]);
  }
  if (x->round_ops)
    for (int32_t f = 0; f < d; ++f) dqrow[f] = bf16_round_d(dqrow[f]);
  x->delta[item] = delta;
  free(P);
}

int orc_bwd_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                     const int32_t* rows, int32_t n, double* o, double* delta, double* dq,
                     int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !qheads || !rows || !o || !delta || !dq) return -1;
  for (int32_t i = 0; i < n; ++i) {
    if (qheads[i] < 0 || qheads[i] >= p->batch * p->heads_q) return -2;
    if (rows[i] < 0 || rows[i] >= p->seqlen) return -2;
  }
  bwdrow_ctx c = {p, q, k, v, dout, qheads, rows, o, delta, dq, NULL, 0};
  run_pool(bwdrow_item, &c, n, nthreads);
  return 0;
}

/* Single rows replayed at the method's rounding points (see orc_bwd_emu). */
int orc_bwd_rows_emu(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                     const int32_t* rows, int32_t n, const double* o_in, int32_t round_ops,
                     double* delta, double* dq, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !qheads || !rows || !delta || !dq) return -1;
  for (int32_t i = 0; i < n; ++i) {
    if (qheads[i] < 0 || qheads[i] >= p->batch * p->heads_q) return -2;
    if (rows[i] < 0 || rows[i] >= p->seqlen) return -2;
  }
  double* otmp = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)p->head_dim);
  bwdrow_ctx c = {p, q, k, v, dout, qheads, rows, otmp, delta, dq, o_in, round_ops};
  run_pool(bwdrow_item, &c, n, nthreads);
  free(otmp);
  return 0;
}

/* The other form of the backward's delta, written out as the pages give it:
 * delta_i = sum_j P_ij dP_ij with P the exact softmax row and dP_ij =
 * dO_i . V_j ([R] method, paper §3.2: rowsum(dP∘P) is mathematically the
 * same as rowsum(dO∘O); [S] "Key claims").  All in double. */
typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v, *dout;
  const int32_t *qheads, *rows;
  double* delta;
} deltadp_ctx;

static void deltadp_item(void* c, int32_t item) {
  deltadp_ctx* x = (deltadp_ctx*)c;
  const orc_problem* p = x->p;
  int32_t qh = x->qheads[item], i = x->rows[item];
  int32_t d = p->head_dim;
  const uint16_t* qi = x->q + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* doi = x->dout + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  const uint16_t* V = x->v + kv_head_offset(p, qh);
  int32_t n = visible(p, i);
  double* P = (double*)malloc(sizeof(double) * (size_t)n);
  double mx = -INFINITY;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = (double)p->alpha * dot_bf16(qi, K + (size_t)j * d, d);
    if (P[j] > mx) mx = P[j];
  }
  double z = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = exp(P[j] - mx);
    z += P[j];
  }
  double delta = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    double dp = dot_bf16(doi, V + (size_t)j * d, d);
    delta += (P[j] / z) * dp;
  }
  x->delta[item] = delta;
  free(P);
}

int orc_delta_dp_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                          const int32_t* rows, int32_t n, double* delta, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !qheads || !rows || !delta) return -1;
  for (int32_t i = 0; i < n; ++i) {
    if (qheads[i] < 0 || qheads[i] >= p->batch * p->heads_q) return -2;
    if (rows[i] < 0 || rows[i] >= p->seqlen) return -2;
  }
  deltadp_ctx c = {p, q, k, v, dout, qheads, rows, delta};
  run_pool(deltadp_item, &c, n, nthreads);
  return 0;
}

/* Row sums of dS for a given delta, written out: sum_j P_ij (dP_ij -
 * delta_i) with P the exact softmax row and dP_ij = dO_i . V_j, and the
 * magnitude sum_j P_ij |dP_ij - delta_i| of its terms.  [R] "Core idea",
 * equations (paper Eq. 1-2): dS = alpha P∘(dP - delta); the rows of P sum to
 * one, so the row sum is rowsum(dP∘P) - delta (zero for the exact delta).
 * All in double; alpha is left out. */
typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v, *dout;
  const int32_t *qheads, *rows;
  const double* delta_in;
  double *dsum, *wsum;
} dsum_ctx;

static void dsum_item(void* c, int32_t item) {
  dsum_ctx* x = (dsum_ctx*)c;
  const orc_problem* p = x->p;
  int32_t qh = x->qheads[item], i = x->rows[item];
  int32_t d = p->head_dim;
  const uint16_t* qi = x->q + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* doi = x->dout + q_head_offset(p, qh) + (size_t)i * d;
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  const uint16_t* V = x->v + kv_head_offset(p, qh);
  int32_t n = visible(p, i);
  double* P = (double*)malloc(sizeof(double) * (size_t)n);
  double mx = -INFINITY;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = (double)p->alpha * dot_bf16(qi, K + (size_t)j * d, d);
    if (P[j] > mx) mx = P[j];
  }
  double z = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    P[j] = exp(P[j] - mx);
    z += P[j];
  }
  double sum = 0.0, mag = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    double t = (P[j] / z) * (dot_bf16(doi, V + (size_t)j * d, d) - x->delta_in[item]);
    sum += t;
    mag += fabs(t);
  }
  x->dsum[item] = sum;
  x->wsum[item] = mag;
  free(P);
}

int orc_dsum_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                      const int32_t* rows, int32_t n, const double* delta_in, double* dsum,
                      double* wsum, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !qheads || !rows || !delta_in || !dsum || !wsum) return -1;
  for (int32_t i = 0; i < n; ++i) {
    if (qheads[i] < 0 || qheads[i] >= p->batch * p->heads_q) return -2;
    if (rows[i] < 0 || rows[i] >= p->seqlen) return -2;
  }
  dsum_ctx c = {p, q, k, v, dout, qheads, rows, delta_in, dsum, wsum};
  run_pool(dsum_item, &c, n, nthreads);
  return 0;
}

/* ======================================================================
 * The repeated-maximum guard.
 * [R] "Core idea", the fix (paper §4): a row whose maximum r recurs (within
 * the tie window) takes the shift m = beta*r when r > 0 and m = 0 otherwise;
 * every other row takes m = r.  r = 0 is not covered by the page's two cases;
 * it is read as the "otherwise" branch (m = 0).
 * [S] "Key claims" / "Method" (Algorithm 1): the variant that subtracts an
 * extra eps = 2^-5 from the shift of such rows, m = r + eps.
 * ====================================================================== */

static float guard_shift(const orc_problem* p, float r, int tie) {
  if (!tie || p->guard == ORC_GUARD_NONE) return r;
  if (p->guard == ORC_GUARD_BETA) return (r > 0.0f) ? p->beta * r : 0.0f;
  return r + p->shift_eps;
}

/* Tie test on the running top two: count >= 2 within the window <=>
 * r2 >= r - eps, decided as fl32(r - r2) <= eps. */
static int tie_test(const orc_problem* p, float r, float r2) {
  if (r2 == -INFINITY) return 0;
  return (r - r2) <= p->tie_eps;
}

/* Fp32 scaled logit of the definition: t = fl32(alpha * fl32(s)). */
static float scaled_logit(const orc_problem* p, double s) {
  float sf = (float)s;
  return p->alpha * sf;
}

/* ======================================================================
 * Row statistics (r, r2, tie flag, final m) with certification.
 * The kernel's scaled logits differ from the oracle's by at most delta_j per
 * key; the maximum and the second maximum of a set move by at most the
 * largest such delta, so the tie decision is certain when
 * |fl32(r - r2) - eps| exceeds twice that plus the rounding of t itself.
 * ====================================================================== */

typedef struct {
  const orc_problem* p;
  const orc_schedule* s;
  const uint16_t *q, *k;
  const int32_t* heads;
  float *r, *r2, *m;
  uint8_t *flags, *cert;
  row_split rs;
} stats_ctx;

/* Bound on |t_kernel - t| for one key: alpha times the score bound, plus the
 * fp32 roundings of s and of alpha*s on either side. */
static double logit_error(const orc_problem* p, double sv, double sbound) {
  double a = (double)p->alpha;
  return a * sbound + 3.0 * U24 * fabs(a * sv);
}

static int tie_certain(const orc_problem* p, float r, float r2, double dmax) {
  if (r2 == -INFINITY) return 1;
  double gap = (double)(r - r2) - (double)p->tie_eps;
  double margin = 2.0 * dmax + 2.0 * U24 * (fabs((double)r) + fabs((double)r2));
  return fabs(gap) > margin;
}

static void stats_head(void* c, int32_t item) {
  stats_ctx* x = (stats_ctx*)c;
  const orc_problem* p = x->p;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t qh, i_begin, i_end;
  split_item(x->rs, item, x->heads, N, &qh, &i_begin, &i_end);
  const uint16_t* Q = x->q + q_head_offset(p, qh);
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
  for (int32_t i = i_begin; i < i_end; ++i) {
    int32_t n = visible(p, i);
    float r = -INFINITY, r2 = -INFINITY;
    double dmax = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      double sb;
      double sv = dot_with_bound(x->s, Q + (size_t)i * d, K + (size_t)j * d, d, tmp, &sb);
      float t = scaled_logit(p, sv);
      if (t > r) {
        r2 = r;
        r = t;
      } else if (t > r2) {
        r2 = t;
      }
      double e = logit_error(p, sv, sb);
      if (e > dmax) dmax = e;
    }
    int tie = tie_test(p, r, r2);
    size_t ro = (size_t)qh * N + i;
    if (x->r) x->r[ro] = r;
    if (x->r2) x->r2[ro] = r2;
    if (x->m) x->m[ro] = guard_shift(p, r, tie);
    if (x->flags)
      x->flags[ro] = (uint8_t)((tie ? ORC_ROW_TIE : 0) |
                               ((tie && p->guard != ORC_GUARD_NONE) ? ORC_ROW_GUARD_APPLIED : 0));
    if (x->cert) x->cert[ro] = (uint8_t)tie_certain(p, r, r2, dmax);
  }
  free(tmp);
}

int orc_row_stats(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                  const uint16_t* k, const int32_t* heads, int32_t nheads,
                  float* r, float* r2, float* m, uint8_t* flags,
                  uint8_t* flag_cert, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k) return -1;
  if (!heads_valid(heads, nheads, p->batch * p->heads_q)) return -2;
  int32_t n = heads ? nheads : p->batch * p->heads_q;
  stats_ctx c = {p, s, q, k, heads, r, r2, m, flags, flag_cert, split_rows(n, p->seqlen, nthreads)};
  run_pool(stats_head, &c, n * c.rs.nblk, nthreads);
  return 0;
}

/* ======================================================================
 * Unnormalised output for a given shift, in double (signed-error metric).
 * ====================================================================== */

typedef struct {
  const orc_problem* p;
  const uint16_t *q, *k, *v;
  const float* m;
  const int32_t* heads;
  double *obar, *l;
  row_split rs;
} obar_ctx;

static void obar_head(void* c, int32_t item) {
  obar_ctx* x = (obar_ctx*)c;
  const orc_problem* p = x->p;
  int32_t N = p->seqlen, d = p->head_dim;
  int32_t qh, i_begin, i_end;
  split_item(x->rs, item, x->heads, N, &qh, &i_begin, &i_end);
  const uint16_t* Q = x->q + q_head_offset(p, qh);
  const uint16_t* K = x->k + kv_head_offset(p, qh);
  const uint16_t* V = x->v + kv_head_offset(p, qh);
  double* e = (double*)malloc(sizeof(double) * (size_t)N);
  double alpha = (double)p->alpha;
  for (int32_t i = i_begin; i < i_end; ++i) {
    int32_t n = visible(p, i);
    size_t ro = (size_t)qh * N + i;
    double mi = (double)x->m[ro];
    double l = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      e[j] = exp(alpha * dot_bf16(Q + (size_t)i * d, K + (size_t)j * d, d) - mi);
      l += e[j];
    }
    if (x->obar) {
      /* sum_j e[j] V[j][f] in key order, read row by row */
      double* ob = x->obar + ro * d;
      for (int32_t f = 0; f < d; ++f) ob[f] = 0.0;
      for (int32_t j = 0; j < n; ++j)
        for (int32_t f = 0; f < d; ++f) ob[f] += e[j] * (double)orc_f32_from_bf16(V[(size_t)j * d + f]);
    }
    if (x->l) x->l[ro] = l;
  }
  free(e);
}

int orc_obar_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const float* m, const int32_t* heads,
                 int32_t nheads, double* obar, double* l, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!q || !k || !v || !m) return -1;
  if (!heads_valid(heads, nheads, p->batch * p->heads_q)) return -2;
  int32_t n = heads ? nheads : p->batch * p->heads_q;
  obar_ctx c = {p, q, k, v, m, heads, obar, l, split_rows(n, p->seqlen, nthreads)};
  run_pool(obar_head, &c, n * c.rs.nblk, nthreads);
  return 0;
}

/* ======================================================================
 * Streaming BF16 emulation of the guarded forward.
 *
 * The steps follow the FlashAttention-2 tiling the pages analyse ([R] "Why
 * it matters", paper §2.2; "Points to doubt": the analysed implementation
 * keeps P̄V in bf16) with the guard placed inside the tile loop ([S]
 * "Method": one extra line in the standard tiling that detects a repeated
 * maximum as the row is streamed).  For each key block of the schedule:
 *   1. merge the block's scaled logits into the running (r, r2);
 *   2. decide the tie and the shift m (guard_shift);
 *   3. rescale by c = exp(m_old - m) and add P̄ = exp(t - m), with P̄ rounded
 *      to bf16 as a matrix-core operand: Ō <- c Ō + sum P̄_bf16 V,
 *      accumulated in fp32; in bf16 mode the accumulator is rounded to bf16
 *      after every round_n keys (the analysed code used 512-key blocks) and
 *      after the row's last block ([R] "Core idea", equations: the sum lives
 *      in a wider accumulator and is rounded once, which is what the worked
 *      addition shows);
 *   4. ℓ <- c ℓ + sum P̄ in fp32.
 * At the end O = RNE_bf16(Ō/ℓ).
 *
 * Every rounding whose input is known only up to the kernel's arithmetic
 * error (the fp32 dot products, the hardware exp, the fp32 sums) is
 * certified: the emulated value is declared certain only if the exact
 * pre-rounding value lies farther from a bf16 rounding boundary than that
 * error bound.  An uncertain step makes the rest of the row uncertain.
 * ====================================================================== */

typedef struct {
  const orc_problem* p;
  const orc_schedule* s;
  const uint16_t *q, *k, *v;
  const int32_t* heads;
  double *obar, *o;
  uint8_t* obar_cert;
  double* obar_dev;
  float *m, *l;
  uint8_t *flags, *flag_cert, *ex;
  const int32_t *rows_qh, *rows_i; /* row list mode: item = one (head, row) */
  row_split rs;                     /* otherwise: item = (head, block of rows) */
} emu_ctx;

/* Working state of the emulation of one head: buffers for the row's scores,
 * the step's P̄ operand and Ō with its certification bookkeeping, and the
 * running values of the row being replayed. */
typedef struct {
  const orc_problem* p;
  const orc_schedule* sc;
  const uint16_t *Q, *K, *V;
  int32_t N, d, bn, rn;
  int cert_on;
  double exp_err; /* relative error of the implementation's exponential */
  double under;   /* smallest nonzero result of that exponential */
  /* one row */
  double *sv, *sb; /* exact scores and the bounds on the implementation's */
  float* tv;       /* fp32 scaled logits */
  /* one step (block of keys), indexed by key - j0 */
  double* pb;   /* P̄ as the matrix operand */
  double* pamb; /* how far the implementation's operand may differ */
  double* pex;  /* exact P̄ (MXFP4: before the block scale is known) */
  double* prho; /* relative bound on the implementation's P̄ */
  int* pexp;    /* E4M3 exponents of 2^ks P̄ */
  int* texp;    /* exponents of the FP8 products */
  double* terms;
  /* one feature of Ō: value, bound of the current step, carried deviation,
   * certified */
  double *ob, *obb, *odv;
  uint8_t* oc;
  /* the row's running state */
  float r, r2, m, l32;
  int have_m, dec_cert, val_cert, tie, zero_ambig;
  double m_err; /* bound on |implementation's shift - m| */
  double dmax;  /* largest logit error so far */
  double flush_slack; /* total size of the step's P̄ that may flush to zero */
  int ks, ks_amb;     /* FP8: operand scale exponent, and whether it is uncertain */
  uint8_t exb;
} emu_state;

static const double kLog2eD = 1.4426950408889634;

/* The row's exact scores q_i . k_j, the bounds on the implementation's fp32
 * scores, and the fp32 scaled logits. */
static void emu_scores(emu_state* st, int32_t i, int32_t n) {
  const uint16_t* qi = st->Q + (size_t)i * st->d;
  for (int32_t j = 0; j < n; ++j) {
    if (st->cert_on) {
      st->sv[j] = dot_with_bound(st->sc, qi, st->K + (size_t)j * st->d, st->d, st->terms, &st->sb[j]);
    } else {
      st->sv[j] = dot_bf16(qi, st->K + (size_t)j * st->d, st->d);
      st->sb[j] = 0.0;
    }
    st->tv[j] = scaled_logit(st->p, st->sv[j]);
  }
}

static void emu_row_start(emu_state* st) {
  st->r = -INFINITY;
  st->r2 = -INFINITY;
  st->m = 0.0f;
  st->l32 = 0.0f;
  st->have_m = 0;
  st->dec_cert = st->cert_on;
  st->val_cert = st->cert_on;
  st->tie = 0;
  st->zero_ambig = 0;
  st->m_err = 0.0;
  st->exb = 0;
  st->dmax = 0.0;
  for (int32_t f = 0; f < st->d; ++f) {
    st->ob[f] = 0.0;
    st->obb[f] = 0.0;
    st->odv[f] = 0.0;
    st->oc[f] = (uint8_t)st->cert_on;
  }
}

/* 1. Running top two of the scaled logits over keys j0 .. j1-1. */
static void emu_top_two(emu_state* st, int32_t j0, int32_t j1) {
  for (int32_t j = j0; j < j1; ++j) {
    float t = st->tv[j];
    if (t > st->r) {
      st->r2 = st->r;
      st->r = t;
    } else if (t > st->r2) {
      st->r2 = t;
    }
    double e = logit_error(st->p, st->sv[j], st->sb[j]);
    if (e > st->dmax) st->dmax = e;
  }
}

/* 2. Tie decision and shift after the step; *m_err_new: the bound on the
 * implementation's shift, which comes from its own r, within dmax of this
 * one: m = r, r + eps (slope 1), beta r (slope beta) or 0 (no error). */
static float emu_shift(emu_state* st, double* m_err_new) {
  const orc_problem* p = st->p;
  st->tie = tie_test(p, st->r, st->r2);
  if (st->cert_on && !tie_certain(p, st->r, st->r2, st->dmax)) st->dec_cert = 0;
  float mn = guard_shift(p, st->r, st->tie);
  if (st->tie && p->guard == ORC_GUARD_BETA && st->r == 0.0f) st->exb |= ORC_EX_ZERO_MAX_TIE;
  double slope_m = 1.0;
  if (st->tie && p->guard == ORC_GUARD_BETA) slope_m = st->r > 0.0f ? (double)p->beta : 0.0;
  *m_err_new = st->cert_on ? slope_m * st->dmax * (1.0 + 4.0 * U24) : 0.0;
  return mn;
}

/* 3a. Rescale the running sums by c = exp(m_old - m_new), then take the new
 * shift. */
static void emu_rescale(emu_state* st, float mn, double m_err_new) {
  if (st->have_m && mn != st->m) {
    if (mn < st->m) st->exb |= ORC_EX_SHIFT_DECREASED;
    double cexact = exp((double)st->m - (double)mn);
    /* bound for an fp32 evaluation: the argument (m_old - m_new) log2 e
     * formed in fp32 and passed to a base-2 exponential of relative
     * error exp_err, the product c Ō rounded to fp32 */
    double dm2 = fabs((double)st->m - (double)mn) * kLog2eD;
    double rho_c = log(2.0) * (2.0 * U24 * dm2) + st->exp_err + st->m_err + m_err_new;
    /* the same exp flushes a result below the threshold to zero */
    if (cexact <= st->under * (1.0 + 4.0 * rho_c)) {
      if (cexact >= st->under * (1.0 - 4.0 * rho_c)) st->zero_ambig = 1;
      cexact = (cexact < st->under) ? 0.0 : cexact;
    }
    float c32 = (float)cexact;
    if (isinf(c32)) st->exb |= ORC_EX_RESCALE_OVERFLOW;
    for (int32_t f = 0; f < st->d; ++f) {
      st->ob[f] = cexact * st->ob[f];
      st->obb[f] = st->obb[f] * cexact * (1.0 + rho_c) + fabs(st->ob[f]) * (rho_c + U24);
      st->odv[f] = st->odv[f] * cexact * (1.0 + rho_c);
    }
    st->l32 = c32 * st->l32;
  }
  st->m = mn;
  st->m_err = m_err_new;
  st->have_m = 1;
}

/* FP8 product: the operand scale 2^ks of the step (row scale), or 2^8
 * (fixed).  The row scale is an integer decided by floating point, so it is
 * taken in the implementation's precision (fp32: floor(fl32(fl32(r - m)
 * log2 e))); ks_amb: the implementation's r may lie on the other side of an
 * integer step. */
static void emu_fp8_scale(emu_state* st) {
  const orc_problem* p = st->p;
  st->ks = 8;
  st->ks_amb = 0;
  if (st->sc->pv_fp8 != 1) return;
  const float d2 = (st->r - st->m) * (float)1.44269504088896340736;
  const float fd = floorf(d2);
  st->ks = 7 - (int)(fd >= -113.0f ? fd : -113.0f);
  double slope = p->guard == ORC_GUARD_BETA ? fabs((double)p->beta - 1.0) : 1.0;
  double slack = 1.01 * slope * kLog2eD * st->dmax +
                 8.0 * U24 * kLog2eD * (fabs((double)st->r) + fabs((double)st->m));
  /* where the shift is r itself, r - m = 0 on both sides */
  if (st->m != st->r && ((double)d2 - (double)fd <= slack || (double)fd + 1.0 - (double)d2 <= slack))
    st->ks_amb = 1;
  if (st->ks_amb && st->cert_on) st->val_cert = 0;
}

static void emu_note_pbar_one(emu_state* st, double pbv) {
  if (pbv == 1.0) {
    if (st->tie) st->exb |= ORC_EX_PBAR_ONE_TIED;
    if (!st->tie) st->exb |= ORC_EX_PBAR_ONE_PRE_TIE;
  }
}

/* 3b. P̄ = exp(t - m) for keys j0 .. j1-1 as the matrix operand: rounded to
 * bf16, or 2^ks P̄ rounded to E4M3 (MXFP4: emu_mx_pbar, once the block
 * scales are known); 4. the fp32 denominator ℓ, the sum of the fp32 P̄. */
static void emu_pbar(emu_state* st, int32_t j0, int32_t j1) {
  const orc_schedule* sc = st->sc;
  const double alpha = (double)st->p->alpha;
  const double m = (double)st->m;
  const double kscale = ldexp(1.0, st->ks);
  st->flush_slack = 0.0;
  for (int32_t j = j0; j < j1; ++j) {
    const int32_t u = j - j0;
    double xe = alpha * st->sv[j] - m;
    double pbar = exp(xe);
    /* bound for an fp32 evaluation: the argument s alpha log2 e - m log2 e
     * formed in fp32 (one fused step) and passed to a base-2
     * exponential of relative error exp_err */
    double x2 = xe * kLog2eD;
    double err_x2 = kLog2eD * alpha * st->sb[j] * (1.0 + U24) + kLog2eD * st->m_err +
                    U24 * (fabs(alpha * st->sv[j] * kLog2eD) + fabs(m * kLog2eD) + fabs(x2));
    double rho = log(2.0) * err_x2 + st->exp_err;
    double pbv;
    st->pamb[u] = 0.0;
    st->pex[u] = pbar < st->under ? 0.0 : pbar;
    st->prho[u] = rho;
    if (sc->pv_mxfp4) {
      pbv = 0.0; /* set by emu_mx_pbar */
      if (pbar <= st->under * (1.0 + 4.0 * rho)) {
        st->pex[u] = 0.0;
        if (pbar >= st->under * (1.0 - 4.0 * rho)) st->zero_ambig = 1;
        st->flush_slack += 2.0 * pbar;
      }
    } else if (pbar <= st->under * (1.0 + 4.0 * rho)) {
      /* at or below the flush threshold: the implementation gives 0 or a
       * tiny value; take 0 and count the whole size as uncertainty */
      pbv = 0.0;
      if (pbar >= st->under * (1.0 - 4.0 * rho)) st->zero_ambig = 1;
      st->flush_slack += 2.0 * pbar;
    } else if (sc->pv_fp8) {
      /* FP8 operand: P̄ * 2^ks rounded to E4M3, scaled back (exact) */
      const double ps = pbar * kscale;
      pbv = orc_e4m3_round(ps) / kscale;
      if (st->cert_on && orc_e4m3_boundary_distance(ps) <= (rho + 2.0 * U24) * ps) {
        st->val_cert = 0;
        st->pamb[u] = orc_e4m3_ulp(ps * (1.0 + rho)) / kscale; /* a neighbour */
      }
      /* another scale changes the rounding only among the subnormals */
      if (st->cert_on && st->ks_amb && ps < 0x1p-5) st->pamb[u] = fmax(st->pamb[u], 0x1p-9 / kscale * 2.0);
    } else {
      pbv = (double)orc_f32_from_bf16(orc_bf16_from_f64(pbar));
      /* a P̄ next to a rounding boundary may take the neighbouring bf16
       * value in the implementation: that one step, times |V|, joins each
       * element's bound, so only elements that stay clear of a boundary by
       * it are certified */
      if (st->cert_on && orc_bf16_boundary_distance(pbar) <= (rho + 2.0 * U24) * pbar)
        st->pamb[u] = orc_bf16_ulp(pbar * (1.0 + rho));
    }
    st->pexp[u] = pbv != 0.0 ? e4m3_exponent(pbv * kscale) : 0;
    emu_note_pbar_one(st, pbv);
    st->pb[u] = pbv;
    /* 4. fp32 denominator: sum of the fp32 P̄ (sequential order here) */
    float p32 = (pbar < st->under) ? 0.0f : (float)pbar;
    st->l32 = st->l32 + p32;
  }
}

/* MXFP4 operand: the step's keys in two blocks of 32 consecutive keys (OCP
 * MX: a block is 32 consecutive elements along the contraction), each with
 * the scale 2^(floor(log2 amax) - 2) of its largest P̄ (or ceil). */
static void emu_mx_pbar(emu_state* st, int32_t j0, int32_t j1) {
  const orc_schedule* sc = st->sc;
  for (int h = 0; h < 2; ++h) {
    double amax = 0.0, rmax = 0.0;
    for (int32_t j = j0; j < j1; ++j)
      if (((j - j0) >> 5) == h) {
        amax = fmax(amax, st->pex[j - j0]);
        rmax = fmax(rmax, st->prho[j - j0]);
      }
    int (*sbf)(double) = sc->pv_mxfp4 == 2 ? orc_mx_scale_byte_ceil : orc_mx_scale_byte;
    const int sbyte = sbf(amax);
    const double X = ldexp(1.0, sbyte - 127);
    /* the implementation's amax is within rmax of this one: its scale may
     * be the neighbouring power of two */
    const int s_amb = st->cert_on && amax > 0.0 &&
                      (sbf(amax * (1.0 - rmax - 2.0 * U24)) != sbyte ||
                       sbf(amax * (1.0 + rmax + 2.0 * U24)) != sbyte);
    if (s_amb) st->val_cert = 0;
    for (int32_t j = j0; j < j1; ++j) {
      const int32_t u = j - j0;
      if ((u >> 5) != h) continue;
      const double y = st->pex[u] / X;
      const double pbv = orc_e2m1_round(y) * X;
      if (st->cert_on && st->pex[u] > 0.0 &&
          orc_e2m1_boundary_distance(y) <= (st->prho[u] + 2.0 * U24) * y) {
        st->val_cert = 0;
        st->pamb[u] = orc_e2m1_spacing(y * (1.0 + st->prho[u])) * X;
      }
      if (s_amb) st->pamb[u] = fmax(st->pamb[u], 4.0 * X);
      emu_note_pbar_one(st, pbv);
      st->pb[u] = pbv;
    }
  }
}

/* The step's products P̄_j V_jf for feature f as they enter the sum (V
 * rounded as the product's format takes it); *vmax: the largest |V|
 * operand, *amb: how far the operand ambiguity of P̄ can move the sum. */
static void emu_terms(emu_state* st, int32_t f, int32_t j0, int32_t j1, double* vmax, double* amb) {
  const orc_schedule* sc = st->sc;
  const int32_t d = st->d;
  double vx[2] = {1.0, 1.0}; /* MXFP4: V's scales over the step's keys */
  if (sc->pv_mxfp4) {
    /* per feature, over every key of the block that exists: V's operand is
     * one for all query rows, so a row's causal mask cannot enter its scale */
    const int32_t jt = j0 + st->bn < st->N ? j0 + st->bn : st->N;
    double va[2] = {0.0, 0.0};
    for (int32_t j = j0; j < jt; ++j) {
      const int h = (j - j0) >> 5;
      va[h] = fmax(va[h], fabs((double)orc_f32_from_bf16(st->V[(size_t)j * d + f])));
    }
    for (int h = 0; h < 2; ++h)
      vx[h] = ldexp(1.0, (sc->pv_mxfp4 == 2 ? orc_mx_scale_byte_ceil(va[h]) : orc_mx_scale_byte(va[h])) - 127);
  }
  *vmax = 0.0;
  *amb = 0.0;
  for (int32_t j = j0; j < j1; ++j) {
    const int32_t u = j - j0;
    double vv = (double)orc_f32_from_bf16(st->V[(size_t)j * d + f]);
    if (sc->pv_mxfp4) {
      const double X = vx[u >> 5];
      vv = orc_e2m1_round(vv / X) * X;
    }
    if (sc->pv_fp8) {
      vv = orc_e4m3_round(vv); /* the FP8 V operand */
      st->texp[u] = vv != 0.0 ? st->pexp[u] + e4m3_exponent(vv) : 0;
    }
    st->terms[u] = st->pb[u] * vv; /* exact: 8-bit x 8-bit mantissas */
    *vmax = fmax(*vmax, fabs(vv));
    *amb += st->pamb[u] * fabs(vv);
  }
}

/* 3c, FA2 as tensor operations: the step's own product sum rounded to bf16,
 * then added to the rescaled Ō and rounded again (every step is a rounding
 * point); a P̄ next to a rounding boundary may take the neighbouring value,
 * which moves the step's sum by up to amb. */
static void emu_obar_block_bf16(emu_state* st, int32_t f, int32_t nt, double vmax, double amb) {
  dd_t bacc = {0.0, 0.0};
  for (int32_t j = 0; j < nt; ++j) dd_add(&bacc, st->terms[j]);
  double bexact = bacc.hi + bacc.lo;
  double bb = st->cert_on ? chain_bound(st->sc, 0.0, st->terms, nt) + st->flush_slack * vmax + amb : 0.0;
  uint16_t bh = dd_to_bf16(bacc);
  double bv = (double)orc_f32_from_bf16(bh);
  dd_t sum = {0.0, 0.0};
  dd_add(&sum, st->ob[f]);
  dd_add(&sum, bv);
  double sexact = sum.hi + sum.lo;
  uint16_t hb = dd_to_bf16(sum);
  const int bsame = st->dec_cert && st->val_cert && orc_bf16_boundary_distance(bexact) > bb;
  const int same = bsame && orc_bf16_boundary_distance(sexact) > st->obb[f] + 2.0 * U24 * fabs(sexact);
  if (!same) st->oc[f] = 0;
  /* deviation of the implementation's Ō from this one: the carried part,
   * the rescale and the step's own (bb, plus a bf16 step if its rounding
   * may differ), then a step of the sum's rounding */
  double dv = st->odv[f] + st->obb[f] + (bsame ? 0.0 : bb + orc_bf16_ulp(fabs(bexact) + bb));
  st->odv[f] = (same && st->odv[f] == 0.0) ? 0.0 : dv + orc_bf16_ulp(fabs(sexact) + dv);
  st->ob[f] = (double)orc_f32_from_bf16(hb);
  st->obb[f] = 0.0;
}

/* 3c, streaming: Ō <- cŌ + Σ P̄ V in an fp32 accumulator; in bf16 mode the
 * accumulator is rounded to bf16 at the rounding points. */
static void emu_obar_stream(emu_state* st, int32_t f, int32_t nt, double vmax, double amb, int round_here) {
  const orc_schedule* sc = st->sc;
  /* a P̄ next to a rounding boundary may take the neighbouring value */
  st->obb[f] += amb;
  if (st->cert_on)
    st->obb[f] += (sc->pv_mxfp4 ? chain_bound_mx(sc, st->ob[f], st->terms, nt)
                   : sc->pv_fp8 ? chain_bound_fp8(sc, st->ob[f], st->terms, st->texp, nt, -st->ks)
                                : chain_bound(sc, st->ob[f], st->terms, nt)) +
                  st->flush_slack * vmax;
  dd_t acc = {0.0, 0.0};
  dd_add(&acc, st->ob[f]);
  for (int32_t j = 0; j < nt; ++j) dd_add(&acc, st->terms[j]);
  double exact = acc.hi + acc.lo;
  if (round_here) {
    uint16_t hb = dd_to_bf16(acc);
    const int same = st->dec_cert && st->val_cert && orc_bf16_boundary_distance(exact) > st->obb[f];
    if (!same) st->oc[f] = 0;
    /* both sides round values at most odv + obb apart */
    double dv = st->odv[f] + st->obb[f];
    st->odv[f] = (same && st->odv[f] == 0.0) ? 0.0 : dv + orc_bf16_ulp(fabs(exact) + dv);
    st->ob[f] = (double)orc_f32_from_bf16(hb);
    st->obb[f] = 0.0;
  } else {
    st->ob[f] = exact;
    st->obb[f] += 0x1p-52 * fabs(exact);
    if (sc->obar_fp32) st->oc[f] = 0; /* no bit claim in fp32 mode */
  }
}

/* The row's outputs: flags and O = RNE_bf16(fl32(Ō / ℓ)). */
static void emu_row_out(const emu_state* st, const emu_ctx* x, size_t ro) {
  const orc_problem* p = st->p;
  uint8_t fl = 0;
  if (st->tie) fl |= ORC_ROW_TIE;
  if (st->tie && p->guard != ORC_GUARD_NONE) fl |= ORC_ROW_GUARD_APPLIED;
  if (st->l32 == 0.0f) fl |= ORC_ROW_ZERO_DENOM;
  if (x->flags) x->flags[ro] = fl;
  if (x->flag_cert) x->flag_cert[ro] = (uint8_t)(st->dec_cert && !st->zero_ambig);
  if (x->ex) x->ex[ro] = st->exb;
  if (x->m) x->m[ro] = st->m;
  if (x->l) x->l[ro] = st->l32;
  for (int32_t f = 0; f < st->d; ++f) {
    size_t eo = ro * (size_t)st->d + f;
    if (x->obar) x->obar[eo] = st->ob[f];
    if (x->obar_cert) x->obar_cert[eo] = st->oc[f];
    /* bound on |implementation's Ō - this Ō| (certifying runs; infinite
     * where the shift decision itself is uncertain) */
    if (x->obar_dev) x->obar_dev[eo] = !st->cert_on ? NAN : st->dec_cert ? st->odv[f] + st->obb[f] : INFINITY;
    if (x->o) {
      float q32 = (float)st->ob[f] / st->l32;
      x->o[eo] = (double)orc_f32_from_bf16(orc_bf16_from_f32(q32));
    }
  }
}

static void emu_head(void* c, int32_t item) {
  emu_ctx* x = (emu_ctx*)c;
  const orc_problem* p = x->p;
  const orc_schedule* sc = x->s;
  const int32_t N = p->seqlen, d = p->head_dim;
  int32_t qh, i_begin, i_end;
  if (x->rows_qh) { /* one listed row; outputs indexed by the list position */
    qh = x->rows_qh[item];
    i_begin = x->rows_i[item];
    i_end = i_begin + 1;
  } else {
    split_item(x->rs, item, x->heads, N, &qh, &i_begin, &i_end);
  }
  emu_state st;
  memset(&st, 0, sizeof(st));
  st.p = p;
  st.sc = sc;
  st.Q = x->q + q_head_offset(p, qh);
  st.K = x->k + kv_head_offset(p, qh);
  st.V = x->v + kv_head_offset(p, qh);
  st.N = N;
  st.d = d;
  st.bn = sc->block_n > 0 ? sc->block_n : N;
  st.rn = sc->round_n > 0 ? sc->round_n : st.bn;
  st.cert_on = sc->certify != 0;
  st.exp_err = sc->exp_rel_err > 0 ? sc->exp_rel_err : 4.0 * U24;
  st.under = sc->ftz ? 0x1p-126 : 0x1p-149;
  const int32_t bn = st.bn;
  st.sv = (double*)malloc(sizeof(double) * (size_t)N);
  st.sb = (double*)malloc(sizeof(double) * (size_t)N);
  st.tv = (float*)malloc(sizeof(float) * (size_t)N);
  st.pb = (double*)malloc(sizeof(double) * (size_t)bn);
  st.ob = (double*)malloc(sizeof(double) * (size_t)d);
  st.obb = (double*)malloc(sizeof(double) * (size_t)d);
  st.odv = (double*)malloc(sizeof(double) * (size_t)d);
  st.pamb = (double*)malloc(sizeof(double) * (size_t)bn);
  st.pexp = (int*)malloc(sizeof(int) * (size_t)bn);
  st.texp = (int*)malloc(sizeof(int) * (size_t)bn);
  st.pex = (double*)malloc(sizeof(double) * (size_t)bn);
  st.prho = (double*)malloc(sizeof(double) * (size_t)bn);
  st.terms = (double*)malloc(sizeof(double) * (size_t)(bn > d ? bn : d));
  st.oc = (uint8_t*)malloc((size_t)d);

  for (int32_t i = i_begin; i < i_end; ++i) {
    const int32_t n = visible(p, i);
    emu_scores(&st, i, n);
    emu_row_start(&st);
    for (int32_t j0 = 0; j0 < n; j0 += bn) {
      const int32_t j1 = j0 + bn < n ? j0 + bn : n;
      emu_top_two(&st, j0, j1);                      /* 1 */
      double m_err_new;
      const float mn = emu_shift(&st, &m_err_new);   /* 2 */
      emu_rescale(&st, mn, m_err_new);               /* 3a */
      emu_fp8_scale(&st);
      emu_pbar(&st, j0, j1);                         /* 3b, 4 */
      if (sc->pv_mxfp4) emu_mx_pbar(&st, j0, j1);
      /* 3c: rounded after every round_n keys and after the row's last step */
      const int round_here = !sc->obar_fp32 && ((j1 % st.rn) == 0 || j1 == n);
      for (int32_t f = 0; f < d; ++f) {
        double vmax, amb;
        emu_terms(&st, f, j0, j1, &vmax, &amb);
        if (sc->block_bf16 && !sc->obar_fp32)
          emu_obar_block_bf16(&st, f, j1 - j0, vmax, amb);
        else
          emu_obar_stream(&st, f, j1 - j0, vmax, amb, round_here);
      }
    }
    emu_row_out(&st, x, x->rows_qh ? (size_t)item : (size_t)qh * N + i);
  }
  free(st.sv);
  free(st.sb);
  free(st.tv);
  free(st.pb);
  free(st.ob);
  free(st.obb);
  free(st.odv);
  free(st.pamb);
  free(st.pexp);
  free(st.texp);
  free(st.pex);
  free(st.prho);
  free(st.terms);
  free(st.oc);
}

int orc_fwd_emu(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                const uint16_t* k, const uint16_t* v, const int32_t* heads,
                int32_t nheads, double* obar, uint8_t* obar_cert, double* obar_dev,
                double* o, float* m, float* l, uint8_t* flags, uint8_t* flag_cert,
                uint8_t* ex, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!s || !q || !k || !v) return -1;
  if (s->block_n < 0 || s->round_n < 0) return -4;
  if (s->block_n > 0 && s->round_n > 0 && s->round_n % s->block_n != 0) return -4;
  if (!heads_valid(heads, nheads, p->batch * p->heads_q)) return -2;
  int32_t n = heads ? nheads : p->batch * p->heads_q;
  emu_ctx c = {p, s, q, k, v, heads, obar, o, obar_cert, obar_dev, m, l, flags, flag_cert, ex, NULL, NULL,
               split_rows(n, p->seqlen, nthreads)};
  run_pool(emu_head, &c, n * c.rs.nblk, nthreads);
  return 0;
}

int orc_fwd_emu_rows(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v, const int32_t* qheads,
                     const int32_t* rows, int32_t n, double* o, float* m, float* l,
                     uint8_t* flags, int32_t nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!s || !q || !k || !v || !qheads || !rows) return -1;
  if (s->block_n < 0 || s->round_n < 0) return -4;
  if (s->block_n > 0 && s->round_n > 0 && s->round_n % s->block_n != 0) return -4;
  for (int32_t i = 0; i < n; ++i) {
    if (qheads[i] < 0 || qheads[i] >= p->batch * p->heads_q) return -2;
    if (rows[i] < 0 || rows[i] >= p->seqlen) return -2;
  }
  orc_schedule s2 = *s;
  s2.certify = 0;
  emu_ctx c = {p, &s2, q, k, v, NULL, NULL, o, NULL, NULL, m, l, flags, NULL, NULL, qheads, rows, {1, 0}};
  run_pool(emu_head, &c, n, nthreads);
  return 0;
}
