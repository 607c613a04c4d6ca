// attn_bwd_common.h -- pieces shared by the two backward kernels
// (attn_bwd_dq.hip, attn_bwd_dkdv.hip).  Not part of the ABI.
#pragma once
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// The log2-domain shift of a row: P = exp(t - m) / l = exp2(t*log2(e) - lse2).
// A row whose every weight underflowed (l == 0) keeps P = NaN, as 0 * (1/0)
// gives.
__device__ __forceinline__ float row_lse2(float m, float l) {
  return l > 0.0f ? __builtin_fmaf(m, kLog2e, __builtin_log2f(l)) : __builtin_nanf("");
}

}  // namespace
}  // namespace attn
