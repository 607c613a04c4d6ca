/*
 * attn.h -- C ABI of the guarded BF16 FlashAttention library (gfx950).
 *
 * The operation is softmax attention O = softmax(alpha * Q K^T) V computed
 * tile by tile with an online softmax and an unnormalised accumulator
 * Ō = P̄ V, and its gradient, with the repeated-row-maximum guard of
 *   [R] "BF16 플래시 어텐션은 왜 수천 스텝 뒤에 무너질까" (priors.kr review of
 *       Qiu & Yao, "Why Low-Precision Transformer Training Fails: An Analysis
 *       on Flash Attention"), and
 *   [S] "Why Low-Precision Transformer Training Fails: An Analysis on Flash
 *       Attention" (bud-325.pages.dev summary).
 * Each entry point below names the passage that defines it.
 *
 * Conventions shared by every entry point
 *   - A tensor is indexed [batch][heads][seqlen][head_dim] with head_dim
 *     contiguous; Q, O, dO, dQ have heads_q heads, K, V, dK, dV have heads_kv
 *     heads.  Element (b, h, n, f) of tensor X lives at
 *     X + b*X_stride.batch + h*X_stride.head + n*X_stride.row + f (elements),
 *     so head-transposed views of a projection output ([batch][seqlen]
 *     [heads][head_dim], or one third of a fused [batch][seqlen][3][heads]
 *     [head_dim] QKV output, as in the GPT-2 attention layers the pages
 *     train: [R] "Core idea" -> method, paper §3.1) are passed without a
 *     copy.  A stride triple of zeros selects the dense layout (batch =
 *     heads*seqlen*head_dim, head = seqlen*head_dim, row = head_dim).
 *     Per-row vectors (row_m, row_l, row_flags, delta, row_max, row_dsum)
 *     and the optional Ō output are always dense [batch][heads_q][seqlen]
 *     (x head_dim).
 *   - Strides: every stride >= 0 and a multiple of 8 elements (16 bytes);
 *     row >= head_dim; (seqlen + 256) * row * 2 < 2^31 (one head's rows,
 *     in bytes, addressed with 32-bit offsets).  Output tensors (o, dq, dk,
 *     dv) must not overlap each other or any input; inputs may share memory
 *     (q, k and v may be views of one buffer).
 *   - Every pointer is a device pointer owned by the caller; the library
 *     neither allocates nor frees, keeps no state between calls, never
 *     synchronises and never prints.  Tensor pointers must be 16-byte
 *     aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; a device fault surfaces at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is enqueued: a bad argument
 *     returns a negative ATTN_E_* code and enqueues nothing.
 *   - Calls on different streams with disjoint outputs may run concurrently.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 12

/* attn_params.flags */
#define ATTN_CAUSAL 0x1u          /* key j visible to query i iff j <= i       */
#define ATTN_GUARD_NONE 0x0u      /* shift m = row max r (plain online softmax) */
#define ATTN_GUARD_BETA 0x2u      /* tie rows: m = beta*r if r > 0, else 0      */
#define ATTN_GUARD_EPS 0x4u       /* tie rows: m = r + shift_eps                */
#define ATTN_GUARD_MASK 0x6u
#define ATTN_OBAR_FP32 0x8u       /* keep Ō in fp32 (default: bf16 per block)   */
#define ATTN_DELTA_DP 0x10u       /* backward: delta = rowsum(dP∘P), not dO∘O   */
/* forward rounding schedule (at most one; default: the streaming kernel) */
#define ATTN_SCHED_FA2_OPS 0x20u  /* 512-key blocks, bf16 block product P̄V     */
#define ATTN_SCHED_UNTILED 0x40u  /* one block holding the whole row            */
#define ATTN_SCHED_MASK 0x60u
/* forward: the P̄V product in FP8 E4M3 (streaming schedule only)          */
#define ATTN_PV_FP8 0x80u
#define ATTN_PV_FP8_FIXED 0x100u  /* with ATTN_PV_FP8: operand scale 2^8     */
/* forward: the P̄V product in MXFP4 (streaming schedule only, not with FP8) */
#define ATTN_PV_MXFP4 0x200u
#define ATTN_PV_MX_CEIL 0x400u    /* with ATTN_PV_MXFP4: scales from ceil(log2) */

/* per-row flag bits written by attn_fwd */
#define ATTN_ROW_TIE 0x1u           /* the row maximum recurs within tie_eps   */
#define ATTN_ROW_ZERO_DENOM 0x2u    /* ℓ == 0 (every P̄ underflowed): O is NaN */
#define ATTN_ROW_GUARD_APPLIED 0x4u /* a guarded shift was used for the row    */

/* return codes */
#define ATTN_OK 0
#define ATTN_E_NULL (-1)        /* a required pointer is NULL                   */
#define ATTN_E_SHAPE (-2)       /* non-positive size, heads_q % heads_kv != 0,
                                   (seqlen+256)*row_stride*2 >= 2^31, or more
                                   than 2^24 - 1 workgroups of 128 rows
                                   (batch*heads_q*ceil(seqlen/128))          */
#define ATTN_E_UNSUPPORTED (-3) /* head_dim not 64/128, misaligned pointer,
                                   stride negative, not a multiple of 8
                                   elements, or a row stride < head_dim      */
#define ATTN_E_PARAM (-4)       /* bad beta/tie_eps/shift_eps/flags/scale       */
#define ATTN_E_HIP (-6)         /* the HIP runtime refused a launch             */

/* Element strides of one [batch][heads][seqlen][head_dim] tensor (the
 * head_dim stride is 1).  {0, 0, 0} selects the dense layout. */
typedef struct {
  int64_t batch, head, row;
} attn_strides;

typedef struct {
  int32_t batch;     /* > 0                                                  */
  int32_t heads_q;   /* > 0, multiple of heads_kv (grouped-query attention)  */
  int32_t heads_kv;  /* > 0; query head h reads KV head h / (heads_q/heads_kv) */
  int32_t seqlen;    /* > 0; queries and keys have the same length           */
  int32_t head_dim;  /* 64 or 128                                            */
  float softmax_scale; /* alpha; <= 0 selects fl32(1/sqrt(head_dim))          */
  float beta;        /* beta-guard multiplier, > 1 (the pages use 2..8)      */
  float tie_eps;     /* tie window, >= 0: tie iff fl32(r - r2) <= tie_eps    */
  float shift_eps;   /* eps-guard extra shift, > 0 (the pages use 2^-5)      */
  uint32_t flags;    /* ATTN_CAUSAL | one ATTN_GUARD_* | ATTN_OBAR_FP32 |
                        ATTN_DELTA_DP | one ATTN_SCHED_* | ATTN_PV_FP8 (+
                        ATTN_PV_FP8_FIXED) or ATTN_PV_MXFP4                  */
  /* layouts of the tensors (see the conventions above); zero = dense        */
  attn_strides q_stride, k_stride, v_stride, o_stride;     /* attn_fwd, attn_bwd */
  attn_strides do_stride, dq_stride, dk_stride, dv_stride; /* attn_bwd          */
} attn_params;

/*
 * attn_fwd -- guarded streaming forward.
 * Defines: [R] "Why it matters" (tiled attention, paper §2.2) and "Core
 * idea" equations (O = PV with P̄ = exp(S - m), paper §3.3.2); the guard:
 * [R] "Core idea", the fix (paper §4) and [S] "Method" (Algorithm 1, one
 * extra line in the tiling loop that detects a repeated maximum).
 * Per query row the keys are streamed in blocks of attn_schedule()'s block_n
 * keys.  After each block: (r, r2) = the two largest scaled logits
 * t = fl32(alpha*s) so far; tie = fl32(r - r2) <= tie_eps; m = guard shift
 * of r; Ō <- exp(m_old - m) Ō + sum bf16(exp(t - m)) V, accumulated in fp32;
 * ℓ <- exp(m_old - m) ℓ + sum exp(t - m) in fp32.  Unless ATTN_OBAR_FP32, Ō
 * is rounded to bf16 after every round_n keys and after the row's last
 * block.  Finally O = bf16(Ō/ℓ).
 *   q [B,Hq,N,d] bf16, k/v [B,Hkv,N,d] bf16                (in; q_stride,
 *                                                  k_stride, v_stride)
 *   o [B,Hq,N,d] bf16                                       (out; o_stride)
 *   row_m [B,Hq,N] fp32: the final shift m                  (out, required)
 *   row_l [B,Hq,N] fp32: ℓ relative to row_m                (out, required)
 *   row_flags [B,Hq,N] u8: ATTN_ROW_* bits                  (out, required)
 *   obar_out [B,Hq,N,d]: final Ō, bf16 (or fp32 with ATTN_OBAR_FP32) (nullable)
 *   row_max [B,Hq,N] fp32: r, the row maximum of t          (nullable)
 * row_m and row_l are what attn_bwd needs to recompute P = exp(t - m)/ℓ.
 * Other schedules (the rest as above):
 *   ATTN_SCHED_FA2_OPS: FlashAttention-2 as tensor operations, the
 *     implementation the pages analyse ([R] "Points to doubt": block size
 *     512, the block product P̄V kept in bf16): per 512-key block the
 *     decision and shift over the block, then B = sum P̄_bf16 V (fp32) and
 *     Ō = bf16(cŌ + bf16(B)).
 *   ATTN_SCHED_UNTILED: one block per row ([S] "Key claims": disabling
 *     tiling still fails): the shift from all the row's keys, Ō =
 *     bf16(sum P̄_bf16 V) rounded once.
 * attn_schedule() reports each schedule's block_n / round_n.
 * ATTN_PV_FP8 (streaming schedule only; ATTN_E_PARAM with another): the
 *   open question of the bias with fewer mantissa bits ([R] "Open
 *   questions").  The matrix operands of Ō's product become
 *   e4m3(2^k exp(t - m)) and e4m3(V), OCP E4M3 (bias 7, largest 448) rounded
 *   to nearest even, with k = 7 - floor(fl32(fl32(r - m) * fl32(log2 e)))
 *   per row and block (r the running maximum, m the block's shift): the
 *   row's largest P̄ lands in [128, 256).  With ATTN_PV_FP8_FIXED, k = 8.
 *   The products and their fp32 sums carry 2^k, moved exactly with the
 *   rescale when k changes and removed before Ō is written or divided by
 *   ℓ.  Rounding points of Ō, ℓ (fp32 exp values) and the shift are
 *   unchanged.  V entries must round inside E4M3's range (|V| < 464);
 *   beyond it the result is undefined.  attn_bwd ignores both flags (it
 *   recomputes P in fp32 and reads O as given).
 * ATTN_PV_MXFP4 (streaming schedule only, not with ATTN_PV_FP8): the same
 *   question for the other format the pages name there.  The operands become
 *   MXFP4 in the OCP MX sense: E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 *   negatives) sharing one E8M0 scale X = 2^(floor(log2 amax) - 2) per
 *   block, each element RNE(clamp(v / X, -6, 6)).  A block is 32
 *   consecutive keys, the first or the second half of a 64-key streaming
 *   step -- per query row for P̄, per feature for V (over every key of the
 *   block that exists: V's operand serves every query row, so no row's
 *   causal mask enters its scale).  The scales are applied inside the scaled matrix
 *   instruction; Ō, ℓ and the shift are as in the bf16 path.  With
 *   ATTN_PV_MX_CEIL the scales are 2^(ceil(log2 amax) - 2) instead (amax / X
 *   in (2, 4]: no element saturates; equal to the rule above when amax is a
 *   power of two) -- the rounding-up rule some MX implementations use.
 */
int attn_fwd(const attn_params* p, const void* q, const void* k, const void* v,
             void* o, float* row_m, float* row_l, uint8_t* row_flags,
             void* obar_out, float* row_max, void* stream);

/*
 * attn_bwd -- backward of attn_fwd: attn_bwd_dq then attn_bwd_dkdv.
 * Defines: [R] "Core idea", equations (paper Eq. 1-2: dS = alpha P∘(dP -
 * delta), dQ = dS K, delta = rowsum(dO∘O)) and the summary/method sections
 * (delta computed from the bf16 O, paper §3.2).  The guard is carried by
 * recomputing P = exp(t - row_m) / row_l with the stored shift ([R] the fix:
 * the backward is otherwise unchanged).
 *   q, k, v, o (bf16; q/k/v/o_stride), dout [B,Hq,N,d] bf16 (do_stride),
 *   row_m, row_l from attn_fwd                              (in)
 *   dq [B,Hq,N,d], dk/dv [B,Hkv,N,d] bf16                  (out; dq/dk/
 *                                                  dv_stride)
 *   delta [B,Hq,N] fp32 = rowsum(dO∘O)                      (out, required)
 * With ATTN_DELTA_DP, delta = rowsum(dP∘P) instead: the pages' other form
 * of the same quantity, which never reads the bf16 O ([R] method, paper
 * §3.2: computing it this way also stabilised training; [S] "Key claims").
 * It costs a first sweep over the keys (S and dP once more) in
 * attn_bwd_dq; o is not read and may be NULL.
 *   row_dsum [B,Hq,N] fp32 (out, nullable): sum_j P_ij (dP_ij - delta_i),
 * the row sum of dS without the factor alpha, in fp32 over the fp32 values
 * (before their bf16 rounding as the dQ operand).  In exact arithmetic it is
 * rowsum(dP∘P) - delta: zero with ATTN_DELTA_DP, and minus the error of the
 * low-precision delta otherwise -- the per-token coefficient through which
 * that error enters the query gradient ([R] "Core idea", equations, paper
 * Eq. 1-2).  Not computed (no cost) when NULL.
 * dK and dV sum over the heads_q/heads_kv query heads sharing a KV head.
 * No scratch memory: every output element is written once, by one
 * workgroup, so results are bitwise reproducible.
 */
int attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
             const void* o, const void* dout, const float* row_m, const float* row_l,
             void* dq, void* dk, void* dv, float* delta, float* row_dsum, void* stream);

/* attn_bwd's stages, callable one by one (same arguments and rules), in
 * this order:
 *   attn_bwd_dq: per query row, delta = rowsum(dO∘O) in fp32 from the bf16
 *     O ([R] "Core idea"/method: the delta term, paper §3.2), or with
 *     ATTN_DELTA_DP delta = rowsum(dP∘P) in fp32 from a first sweep over
 *     the row's keys, written to delta; then over every key the row sees,
 *     S, P = exp(t - row_m)/row_l,
 *     dP = dO V^T, dS = P∘(dP - delta) and dQ = alpha dS K ([R] "Core
 *     idea", Eq. 1-2).
 *   attn_bwd_dkdv: per key, over every query row that sees it, the same S,
 *     P, dP and dS from delta (as written by attn_bwd_dq); dV = P^T dO and
 *     dK = alpha dS^T Q ([R] "Core idea", Eq. 1-2).                        */
int attn_bwd_dq(const attn_params* p, const void* q, const void* k, const void* v,
                const void* o, const void* dout, const float* row_m, const float* row_l,
                void* dq, float* delta, float* row_dsum, void* stream);
int attn_bwd_dkdv(const attn_params* p, const void* q, const void* k, const void* v,
                  const void* dout, const float* row_m, const float* row_l,
                  const float* delta, void* dk, void* dv, void* stream);

/*
 * attn_bwd_workspace_bytes -- the device scratch that attn_bwd needs for
 * these params: 0 for every valid parameter set.  The gradient dQ = dS K
 * ([R] "Core idea", equations, paper Eq. 1-2) is usually accumulated from
 * many key blocks into an fp32 workspace; here the dQ kernel finishes each
 * row's dQ in registers and every output element is written once, so no
 * workspace exists.  The query lets a caller that sizes a workspace before
 * the call learn that it needs none.  Returns (size_t)-1 for params that
 * attn_bwd would reject (the same checks).
 */
size_t attn_bwd_workspace_bytes(const attn_params* p);

/*
 * attn_schedule -- the rounding schedule attn_fwd uses for these params, so
 * that a reference can replay it: block_m query rows per workgroup, block_n
 * keys per streaming step (tie decision and shift; 0 = the whole row),
 * round_n keys per bf16 rounding of Ō (bf16 mode; 0 = the whole row),
 * chunk = products per matrix instruction along each bf16 contraction,
 * block_bf16 = 1 when each block's product is rounded to bf16 before it is
 * added to Ō, pv_chunk = products per matrix instruction of the P̄V product
 * (16 in bf16; 64 with ATTN_PV_FP8 or ATTN_PV_MXFP4: one instruction per
 * feature block and 64-key step).  Returns ATTN_OK or an error code for
 * invalid params.  Pointers may be NULL.
 */
int attn_schedule(const attn_params* p, int32_t* block_m, int32_t* block_n,
                  int32_t* round_n, int32_t* chunk, int32_t* block_bf16, int32_t* pv_chunk);

const char* attn_strerror(int code);
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
