// attn_api.cpp -- the C ABI declared in include/attn.h: argument checks,
// kernel selection and launches on the caller's stream.  No allocation, no
// synchronisation, no global state.
#include "attn.h"

#include <cmath>
#include <cstdint>

#include "attn_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float scale_of(const attn_params* p) {
  if (p->softmax_scale > 0.0f) return p->softmax_scale;
  return (float)(1.0 / std::sqrt((double)p->head_dim));
}

// The layout of one tensor with `heads` heads from its strides ({0, 0, 0}:
// dense).  Returns ATTN_OK or the error code of attn.h's stride rules.
int layout_of(const attn_params* p, const attn_strides& s, int heads, attn::Layout* out) {
  const int64_t d = p->head_dim, n = p->seqlen;
  attn_strides t = s;
  if (t.batch == 0 && t.head == 0 && t.row == 0) {
    t.row = d;
    t.head = n * d;
    t.batch = (int64_t)heads * n * d;
  }
  if (t.batch < 0 || t.head < 0 || t.row < 0) return ATTN_E_UNSUPPORTED;
  if (t.batch % 8 != 0 || t.head % 8 != 0 || t.row % 8 != 0) return ATTN_E_UNSUPPORTED;
  if (t.row < d) return ATTN_E_UNSUPPORTED;
  // one head's rows, and the rows a tile copy reads past the end (zeros),
  // are addressed with 32-bit byte offsets
  if ((double)(n + 256) * (double)t.row * 2.0 >= 2147483648.0) return ATTN_E_SHAPE;
  const double last = (double)(p->batch - 1) * t.batch + (double)(heads - 1) * t.head +
                      (double)(n - 1) * t.row + (double)d;
  if (last > 9.0e15) return ATTN_E_SHAPE;
  if (out) {
    out->sb = t.batch;
    out->sh = t.head;
    out->sn = (int)t.row;
  }
  return ATTN_OK;
}

int check_layouts(const attn_params* p) {
  const attn_strides* q_like[] = {&p->q_stride, &p->o_stride, &p->do_stride, &p->dq_stride};
  const attn_strides* kv_like[] = {&p->k_stride, &p->v_stride, &p->dk_stride, &p->dv_stride};
  for (const attn_strides* s : q_like) {
    const int rc = layout_of(p, *s, p->heads_q, nullptr);
    if (rc) return rc;
  }
  for (const attn_strides* s : kv_like) {
    const int rc = layout_of(p, *s, p->heads_kv, nullptr);
    if (rc) return rc;
  }
  return ATTN_OK;
}

int check_params(const attn_params* p) {
  if (!p) return ATTN_E_NULL;
  if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seqlen <= 0 ||
      p->head_dim <= 0)
    return ATTN_E_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return ATTN_E_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return ATTN_E_UNSUPPORTED;
  const uint32_t known =
      ATTN_CAUSAL | ATTN_GUARD_MASK | ATTN_OBAR_FP32 | ATTN_DELTA_DP | ATTN_SCHED_MASK | ATTN_PV_FP8 |
      ATTN_PV_FP8_FIXED | ATTN_PV_MXFP4 | ATTN_PV_MX_CEIL;
  if (p->flags & ~known) return ATTN_E_PARAM;
  if ((p->flags & ATTN_SCHED_MASK) == ATTN_SCHED_MASK) return ATTN_E_PARAM;  // two schedules
  // the FP8 product exists in the streaming kernel only
  if ((p->flags & ATTN_PV_FP8) && (p->flags & ATTN_SCHED_MASK)) return ATTN_E_PARAM;
  if ((p->flags & ATTN_PV_FP8_FIXED) && !(p->flags & ATTN_PV_FP8)) return ATTN_E_PARAM;
  // MXFP4: streaming kernel only, and one low-precision format at a time
  if ((p->flags & ATTN_PV_MXFP4) && (p->flags & (ATTN_SCHED_MASK | ATTN_PV_FP8))) return ATTN_E_PARAM;
  if ((p->flags & ATTN_PV_MX_CEIL) && !(p->flags & ATTN_PV_MXFP4)) return ATTN_E_PARAM;
  const uint32_t g = p->flags & ATTN_GUARD_MASK;
  if (g == ATTN_GUARD_MASK) return ATTN_E_PARAM;  // two guards at once
  if (!std::isfinite(p->softmax_scale)) return ATTN_E_PARAM;
  if (g == ATTN_GUARD_BETA && !(p->beta > 1.0f && std::isfinite(p->beta))) return ATTN_E_PARAM;
  if (!(p->tie_eps >= 0.0f && std::isfinite(p->tie_eps))) return ATTN_E_PARAM;
  if (g == ATTN_GUARD_EPS && !(p->shift_eps > 0.0f && std::isfinite(p->shift_eps))) return ATTN_E_PARAM;
  // rows * head_dim must fit the kernels' index arithmetic; the strides
  // (one head's rows within a 32-bit byte range) are checked per tensor
  const double elems = (double)p->batch * p->heads_q * p->seqlen * p->head_dim;
  if (elems > 9.0e15) return ATTN_E_SHAPE;
  const int lrc = check_layouts(p);
  if (lrc) return lrc;
  // a launch covers at most 2^32 - 1 work-items: 256-thread workgroups of
  // 128 query rows (forward, dQ) or keys (dK/dV, fewer heads)
  const double groups = (double)p->batch * p->heads_q * ((p->seqlen + 127) / 128);
  if (groups > 16777215.0) return ATTN_E_SHAPE;
  return ATTN_OK;
}

int guard_of(uint32_t flags) {
  switch (flags & ATTN_GUARD_MASK) {
    case ATTN_GUARD_BETA: return attn::kGuardBeta;
    case ATTN_GUARD_EPS: return attn::kGuardEps;
    default: return attn::kGuardNone;
  }
}

attn::BwdArgs bwd_args(const attn_params* p, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* row_m, const float* row_l,
                       void* dq, void* dk, void* dv, float* delta) {
  attn::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.row_m = row_m;
  a.row_l = row_l;
  a.delta = delta;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.B = p->batch;
  a.Hq = p->heads_q;
  a.Hkv = p->heads_kv;
  a.N = p->seqlen;
  a.group = p->heads_q / p->heads_kv;
  a.alpha = scale_of(p);
  a.c1 = a.alpha * attn::kLog2e;
  // validated by check_params
  layout_of(p, p->q_stride, p->heads_q, &a.lq);
  layout_of(p, p->k_stride, p->heads_kv, &a.lk);
  layout_of(p, p->v_stride, p->heads_kv, &a.lv);
  layout_of(p, p->o_stride, p->heads_q, &a.lo);
  layout_of(p, p->do_stride, p->heads_q, &a.ldo);
  layout_of(p, p->dq_stride, p->heads_q, &a.ldq);
  layout_of(p, p->dk_stride, p->heads_kv, &a.ldk);
  layout_of(p, p->dv_stride, p->heads_kv, &a.ldv);
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

// O is read by the backward only for delta = rowsum(dO∘O).
bool needs_o(const attn_params* p) { return (p->flags & ATTN_DELTA_DP) == 0; }

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "invalid shape (non-positive size, heads_q not a multiple of heads_kv, or a head too large)";
    case ATTN_E_UNSUPPORTED: return "unsupported head_dim (64 or 128), misaligned tensor pointer or unsupported strides";
    case ATTN_E_PARAM: return "invalid parameter (beta, tie_eps, shift_eps, scale or flags)";
    case ATTN_E_HIP: return "the HIP runtime rejected a kernel launch";
    default: return "unknown error code";
  }
}

size_t attn_bwd_workspace_bytes(const attn_params* p) {
  return check_params(p) == ATTN_OK ? 0 : (size_t)-1;
}

int attn_schedule(const attn_params* p, int32_t* block_m, int32_t* block_n, int32_t* round_n,
                  int32_t* chunk, int32_t* block_bf16, int32_t* pv_chunk) {
  const int rc = check_params(p);
  if (rc) return rc;
  int32_t bn = attn::kFwdBlockN, rn = attn::kFwdRoundN, bb = 0;
  if (p->flags & ATTN_SCHED_FA2_OPS) {
    bn = rn = attn::kFwdOpsBlockN;
    bb = 1;
  } else if (p->flags & ATTN_SCHED_UNTILED) {
    bn = rn = 0;
    bb = 1;
  }
  if (block_m) *block_m = attn::kFwdBlockM;
  if (block_n) *block_n = bn;
  if (round_n) *round_n = rn;
  if (chunk) *chunk = attn::kMfmaK;
  if (block_bf16) *block_bf16 = bb;
  if (pv_chunk) *pv_chunk = (p->flags & (ATTN_PV_FP8 | ATTN_PV_MXFP4)) ? 64 : attn::kMfmaK;
  return ATTN_OK;
}

int attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o,
             float* row_m, float* row_l, uint8_t* row_flags, void* obar_out, float* row_max,
             void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !o || !row_m || !row_l || !row_flags) return ATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (obar_out && !aligned16(obar_out)))
    return ATTN_E_UNSUPPORTED;
  attn::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.row_m = row_m;
  a.row_l = row_l;
  a.row_flags = row_flags;
  a.obar = obar_out;
  a.row_max = row_max;
  a.B = p->batch;
  a.Hq = p->heads_q;
  a.Hkv = p->heads_kv;
  a.N = p->seqlen;
  a.group = p->heads_q / p->heads_kv;
  a.alpha = scale_of(p);
  a.c1 = a.alpha * attn::kLog2e;
  a.beta = p->beta;
  a.tie_eps = p->tie_eps;
  a.shift_eps = p->shift_eps;
  a.pv_fixed_scale = (p->flags & ATTN_PV_FP8_FIXED) != 0;
  a.pv_mx_ceil = (p->flags & ATTN_PV_MX_CEIL) != 0;
  layout_of(p, p->q_stride, p->heads_q, &a.lq);  // validated by check_params
  layout_of(p, p->k_stride, p->heads_kv, &a.lk);
  layout_of(p, p->v_stride, p->heads_kv, &a.lv);
  layout_of(p, p->o_stride, p->heads_q, &a.lo);
  const bool causal = (p->flags & ATTN_CAUSAL) != 0, obar_f32 = (p->flags & ATTN_OBAR_FP32) != 0;
  if (p->flags & ATTN_SCHED_MASK)
    return hip_status(attn::launch_fwd_block(a, p->head_dim, causal, guard_of(p->flags), obar_f32,
                                             (p->flags & ATTN_SCHED_UNTILED) != 0,
                                             (hipStream_t)stream));
  return hip_status(attn::launch_fwd(a, p->head_dim, causal, guard_of(p->flags), obar_f32,
                                     (p->flags & ATTN_PV_FP8) ? 1 : (p->flags & ATTN_PV_MXFP4) ? 2 : 0,
                                     (hipStream_t)stream));
}

int attn_bwd_dkdv(const attn_params* p, const void* q, const void* k, const void* v,
                  const void* dout, const float* row_m, const float* row_l, const float* delta,
                  void* dk, void* dv, void* stream) {
  const int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || !dout || !row_m || !row_l || !delta || !dk || !dv) return ATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dk) ||
      !aligned16(dv))
    return ATTN_E_UNSUPPORTED;
  const attn::BwdArgs a = bwd_args(p, q, k, v, nullptr, dout, row_m, row_l, nullptr, dk, dv,
                                   const_cast<float*>(delta));
  return hip_status(attn::launch_bwd_dkdv(a, p->head_dim, (p->flags & ATTN_CAUSAL) != 0,
                                          (hipStream_t)stream));
}

int attn_bwd_dq(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* row_m, const float* row_l, void* dq, float* delta,
                float* row_dsum, void* stream) {
  const int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || (!o && needs_o(p)) || !dout || !row_m || !row_l || !dq || !delta)
    return ATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o)) ||
      !aligned16(dout) || !aligned16(dq))
    return ATTN_E_UNSUPPORTED;
  attn::BwdArgs a = bwd_args(p, q, k, v, o, dout, row_m, row_l, dq, nullptr, nullptr, delta);
  a.row_dsum = row_dsum;
  return hip_status(attn::launch_bwd_dq(a, p->head_dim, (p->flags & ATTN_CAUSAL) != 0,
                                        (p->flags & ATTN_DELTA_DP) != 0, (hipStream_t)stream));
}

int attn_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* row_m, const float* row_l, void* dq, void* dk,
             void* dv, float* delta, float* row_dsum, void* stream) {
  int rc = check_params(p);
  if (rc) return rc;
  if (!q || !k || !v || (!o && needs_o(p)) || !dout || !row_m || !row_l || !dq || !dk || !dv ||
      !delta)
    return ATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o)) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_E_UNSUPPORTED;
  rc = attn_bwd_dq(p, q, k, v, o, dout, row_m, row_l, dq, delta, row_dsum, stream);
  if (rc) return rc;
  return attn_bwd_dkdv(p, q, k, v, dout, row_m, row_l, delta, dk, dv, stream);
}

}  // extern "C"
