/*
 * oracle.h -- plain, slow, CPU-only reference for guarded BF16 attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only in the tests.
 *
 * Sources (cited by title and section; the pages are prior art, not code):
 *   [R] "BF16 플래시 어텐션은 왜 수천 스텝 뒤에 무너질까" -- priors.kr review of
 *       Qiu & Yao, "Why Low-Precision Transformer Training Fails: An Analysis
 *       on Flash Attention" (ICLR 2026).  Sections used: "Why it matters"
 *       (BF16 format, paper §2.1-2.2), "Core idea" -> intuition / method /
 *       equations (paper §3.2, §3.3.2, Eq. 1-3), the fix (paper §4, App. C),
 *       "Points to doubt" (public PyTorch-ops implementation, App. G) and the
 *       comprehension quiz.
 *   [S] "Why Low-Precision Transformer Training Fails: An Analysis on Flash
 *       Attention" -- bud-325.pages.dev summary.  Sections used: "Key claims",
 *       "Method" (Algorithm 1), "Results" (second addition trace).
 *
 * All tensors are row-major [batch][heads][seqlen][head_dim] with head_dim
 * contiguous.  bf16 values are passed as their 16-bit patterns.  Every entry
 * point returns 0 on success and a negative number on a bad argument.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_GUARD_NONE = 0, ORC_GUARD_BETA = 1, ORC_GUARD_EPS = 2 };
enum { ORC_ROW_TIE = 1, ORC_ROW_ZERO_DENOM = 2, ORC_ROW_GUARD_APPLIED = 4 };
/* per-row exception bits reported by the emulation (not part of the method) */
enum {
  ORC_EX_PBAR_ONE_TIED = 1,   /* bf16(P̄) == 1 in a block that saw the tie  */
  ORC_EX_ZERO_MAX_TIE = 2,     /* tie row with r == 0: m = 0 and P̄_max = 1     */
  ORC_EX_SHIFT_DECREASED = 4,  /* running tie broken later: m went down         */
  ORC_EX_RESCALE_OVERFLOW = 8, /* exp(m_old - m_new) overflowed fp32            */
  ORC_EX_PBAR_ONE_PRE_TIE = 16 /* P̄ == 1 at a first occurrence, before the tie  */
};

typedef struct {
  int32_t batch, heads_q, heads_kv, seqlen, head_dim;
  int32_t causal;     /* 1: key j visible to query i iff j <= i (top-left)    */
  int32_t guard;      /* ORC_GUARD_*                                           */
  float alpha;        /* softmax scale applied to QK^T, as an fp32 value       */
  float beta;         /* beta-guard multiplier (> 1)                           */
  float tie_eps;      /* tie window: repeated max iff r - r2 <= tie_eps        */
  float shift_eps;    /* extra shift of the eps-guard                          */
} orc_problem;

/* The rounding schedule to replay (block_n, round_n, obar_fp32) and the error
 * model of the kernel under test (the other fields), which only decides which
 * emulated values are certain -- never changes them. */
typedef struct {
  int32_t block_n;        /* keys per streaming step (tie decision and shift)  */
  int32_t round_n;        /* bf16 mode: Ō is rounded to bf16 after every
                             round_n keys (a multiple of block_n; 0 = block_n)
                             and after the row's last block                  */
  int32_t obar_fp32;      /* 0: Ō rounded to bf16 (see round_n); 1: fp32      */
  int32_t certify;        /* 0: skip the certification (fast; all cert = 0)   */
  int32_t ftz;            /* 1: exp results below 2^-126 flush to zero         */
  /* Sums computed by the kernel's matrix instructions: a chain of steps, each
   * adding `chunk` terms to the running value C, with the per-step error
   * model of chain_bound() in oracle.c scaled by chunk_err (a safety factor).
   * chunk = 0 means "any order of fp32 additions": n*u*sum|terms|.         */
  int32_t chunk;
  double chunk_err;
  double exp_rel_err;     /* bound on the relative error of the kernel's exp   */
  /* bf16 mode, 1: at each rounding point the product sum of the keys since
   * the previous one is itself rounded to bf16 and then added to the
   * (rescaled) Ō, the sum rounded again -- FA2 written as tensor operations
   * that keep the block product P̄V in bf16 ([R] "Points to doubt": the
   * analysed implementation, block size 512).  Needs round_n == block_n.   */
  int32_t block_bf16;
  /* the P̄V product in FP8 E4M3 -- P̄ * 2^k and V rounded to E4M3 (the
   * scale undone in the sum, exactly); the products are exact.  1: k = 7 -
   * floor(fl32(fl32(r - m) * fl32(log2 e))) per row and block (the row's
   * largest P̄ in [128, 256)); 2: k = 8.  0: bf16 operands.                 */
  int32_t pv_fp8;
  /* 1: the P̄V product in MXFP4 -- P̄ and V in E2M1 elements with one E8M0
   * scale 2^(floor(log2 amax) - 2) per 32 consecutive keys (keys 0..31 and
   * 32..63 of each 64-key step), one scaled matrix instruction per
   * step.  Streaming schedule with block_n = 64 only.  2: the scales from
   * ceil(log2 amax) instead of floor.                                      */
  int32_t pv_mxfp4;
  /* products per matrix instruction of the FP8 P̄V product: 16, or 64 for
   * the scaled 64-product instruction (its group sums add a term to the
   * bound, see chain_bound_fp8 in oracle.c); 0 = 16                       */
  int32_t pv_chunk;
} orc_schedule;

int orc_version(void);

/* ---- BF16 (bfloat16: 8 exponent bits, 7 stored mantissa bits) ---------- */
uint16_t orc_bf16_from_f32(float x);       /* round to nearest, ties to even */
uint16_t orc_bf16_from_f64(double x);      /* direct RNE of a double         */
float orc_f32_from_bf16(uint16_t h);
void orc_bf16_from_f32_array(const float* x, uint16_t* out, int64_t n);
void orc_f32_from_bf16_array(const uint16_t* h, float* out, int64_t n);
double orc_bf16_ulp(double x);             /* spacing of the bf16 grid at |x| */
double orc_bf16_boundary_distance(double x); /* |x - nearest rounding midpoint| */
/* ---- FP8 E4M3 (OCP: bias 7, 3 mantissa bits, max 448, no infinities) ---- */
double orc_e4m3_round(double x);           /* RNE to E4M3 (NaN past 448)      */
double orc_e4m3_ulp(double x);             /* spacing of the E4M3 grid at |x| */
double orc_e4m3_boundary_distance(double x);
/* ---- FP4 E2M1 and MX block scaling (OCP MX) ---- */
double orc_e2m1_round(double y);            /* RNE(clamp(y, -6, 6)) on E2M1   */
double orc_e2m1_spacing(double y);          /* grid spacing at |y|            */
double orc_e2m1_boundary_distance(double y);
int orc_mx_scale_byte(double amax);         /* E8M0 byte of the block scale  */
int orc_mx_scale_byte_ceil(double amax);    /* the same with ceil(log2 amax) */
/* RNE to bf16 of the exact sum of n doubles (the accumulate-then-round step).
 * *exact_out (nullable) receives the exact sum rounded to double.           */
uint16_t orc_bf16_round_of_sum(const double* terms, int32_t n, double* exact_out);

/* ---- FP64 reference (the plain definition) ----------------------------- */
/* O = softmax(alpha QK^T) V in double.  lse[i] = log sum_j exp(alpha s_ij).
 * heads: list of flattened (b*heads_q + h) query heads, or NULL for all.    */
int orc_fwd_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const int32_t* heads, int32_t nheads,
                double* o, double* lse, int32_t nthreads);

/* Backward of softmax attention in double: delta = rowsum(dO∘O),
 * dS = P∘(dP - delta), dQ = alpha dS K, dK = alpha dS^T Q, dV = P^T dO,
 * dK/dV summed over the query heads that share a KV head.
 * kv_heads: list of flattened (b*heads_kv + hk), or NULL for all.  Only the
 * query heads of the listed KV heads are written in o/delta/dq.             */
int orc_bwd_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const uint16_t* dout, const int32_t* kv_heads,
                int32_t nkv, double* o, double* delta, double* dq, double* dk,
                double* dv, int32_t nthreads);

/* The same backward for single query rows: o, delta and dq of row rows[i]
 * of query head qheads[i] (each row's dQ needs only that row).  Outputs are
 * [n, head_dim], [n], [n, head_dim].                                       */
int orc_bwd_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                     const int32_t* rows, int32_t n, double* o, double* delta, double* dq,
                     int32_t nthreads);

/* The backward replayed at the method's rounding points: delta computed from
 * o_in (the forward's bf16 output, [B,Hq,N,d]; NULL = exact O) and, with
 * round_ops, P (for dV) and dS (for dK, dQ) rounded to bf16 as the products'
 * operands and dQ, dK, dV rounded to bf16 as outputs; all else in double.  Measures the method's own deviation from
 * orc_bwd_f64 (its floor), not the kernel's.                               */
int orc_bwd_emu(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const uint16_t* dout, const int32_t* kv_heads,
                int32_t nkv, const double* o_in, int32_t round_ops, double* delta,
                double* dq, double* dk, double* dv, int32_t nthreads);
/* Single-row version: o_in is [n, head_dim] (the rows' O), outputs [n], [n,d]. */
int orc_bwd_rows_emu(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                     const int32_t* rows, int32_t n, const double* o_in, int32_t round_ops,
                     double* delta, double* dq, int32_t nthreads);

/* Error bounds of the kernel's accumulation chains (oracle.c, chain_bound*):
 * c0 + sum(terms) summed by matrix instructions of sc->chunk (bf16) or
 * sc->pv_chunk (FP8: terms are products of E4M3 operands scaled by 2^shift,
 * esum their exponent sums; MXFP4: one instruction) products each. */
double orc_chain_bound(const orc_schedule* sc, double c0, const double* terms, int32_t n);
double orc_chain_bound_fp8(const orc_schedule* sc, double c0, const double* terms,
                           const int32_t* esum, int32_t n, int32_t shift);
double orc_chain_bound_mx(const orc_schedule* sc, double c0, const double* terms, int32_t n);

/* FP64 backward of one KV head (kv_head = b*heads_kv + hk): delta [g, N] for
 * the group's g query heads, dk and dv [N, d] of its keys; parallel over
 * rows, then over blocks of keys.  o_in (nullable, [g, N, d]) and round_ops
 * as in orc_bwd_emu.  Same arithmetic as orc_bwd_f64 / orc_bwd_emu per (i,
 * j): [R] "Core idea", equations (paper Eq. 1-2). */
int orc_bwd_kv_keys(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const uint16_t* dout, int32_t kv_head,
                    const double* o_in, int32_t round_ops, double* delta, double* dk,
                    double* dv, int32_t nthreads);

/* delta_i = sum_j P_ij dP_ij (exact softmax row P, dP_ij = dO_i . V_j) for
 * single rows: row rows[i] of query head qheads[i]; in double.  [R] method
 * (paper §3.2): the form of delta that does not use the low-precision O. */
int orc_delta_dp_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                          const int32_t* rows, int32_t n, double* delta, int32_t nthreads);

/* Row sums of dS for a given delta (delta_in[i] for row i): dsum[i] =
 * sum_j P_ij (dP_ij - delta_in[i]) and wsum[i] = sum_j P_ij |dP_ij -
 * delta_in[i]|, exact softmax P, in double, without alpha.  [R] "Core idea",
 * equations (paper Eq. 1-2). */
int orc_dsum_rows_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const uint16_t* dout, const int32_t* qheads,
                      const int32_t* rows, int32_t n, const double* delta_in, double* dsum,
                      double* wsum, int32_t nthreads);

/* Row statistics on the fp32 scaled logits t = fl32(alpha * fl32(s)):
 * r = max, r2 = second largest (multiset), tie flag, final shift m.
 * flag_cert[i] = 1 when the kernel's score error (orc_schedule's model of
 * its matrix-instruction sums) cannot change the tie decision.             */
int orc_row_stats(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                  const uint16_t* k, const int32_t* heads, int32_t nheads,
                  float* r, float* r2, float* m, uint8_t* flags,
                  uint8_t* flag_cert, int32_t nthreads);

/* Unnormalised output for a given per-row shift m, in double:
 * obar[i,f] = sum_j exp(t_ij - m_i) v_jf and l[i] = sum_j exp(t_ij - m_i),
 * with t the exact scaled logit alpha*s.                                    */
int orc_obar_f64(const orc_problem* p, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const float* m, const int32_t* heads,
                 int32_t nheads, double* obar, double* l, int32_t nthreads);

/* Tile-by-tile emulation of the guarded streaming forward with the rounding
 * points of the schedule, plus certification of every bf16 rounding.
 * Outputs (per query row of the listed heads, in [B,Hq,N(,d)] layout):
 *   obar      final Ō (bf16-valued in bf16 mode), obar_cert 1 = certain
 *   obar_dev  (nullable) bound on |kernel's final Ō - obar| from the error
 *             bounds, carried through every rounding point (one step of the
 *             rounding where it is not certain); +inf on rows whose shift
 *             decision is uncertain; NaN without certification
 *   o         RNE_bf16(Ō/ℓ) as double
 *   m, l      final shift and fp32 denominator; flags = ORC_ROW_* bits
 *   flag_cert 1 = every streaming tie decision of the row (and its zero-
 *             denominator outcome) is certain
 *   ex        ORC_EX_* bits                                                 */
int orc_fwd_emu(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                const uint16_t* k, const uint16_t* v, const int32_t* heads,
                int32_t nheads, double* obar, uint8_t* obar_cert, double* obar_dev,
                double* o, float* m, float* l, uint8_t* flags, uint8_t* flag_cert,
                uint8_t* ex, int32_t nthreads);

/* The same emulation for listed rows only (row rows[i] of query head
 * qheads[i]), without certification; outputs indexed by list position:
 * o [n, head_dim], m, l, flags [n] (each nullable).                        */
int orc_fwd_emu_rows(const orc_problem* p, const orc_schedule* s, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v, const int32_t* qheads,
                     const int32_t* rows, int32_t n, double* o, float* m, float* l,
                     uint8_t* flags, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
