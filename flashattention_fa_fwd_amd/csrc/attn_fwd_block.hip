// attn_fwd_block.hip -- the guarded forward under two other rounding
// schedules, for comparison with the streaming kernel of attn_fwd.hip.
//
// [R] = the priors.kr review "BF16 플래시 어텐션은 왜 수천 스텝 뒤에 무너질까",
// [S] = the bud-325 summary "Why Low-Precision Transformer Training Fails: An
// Analysis on Flash Attention".
//   * FA2_OPS: FlashAttention-2 written as tensor operations, as in the
//     implementation the pages analyse ([R] "Points to doubt": block size
//     512, the unnormalised block product P̄V kept in bf16).  Per block of
//     512 keys: the row maximum (and the repeated-maximum decision) over the
//     block, the shift m and the rescale c = exp(m_old - m); then P̄ =
//     exp(t - m), ℓ = cℓ + sum P̄, and the block product B = sum P̄_bf16 V
//     (fp32 accumulation) rounded to bf16; Ō = bf16(cŌ + bf16(B)).
//   * UNTILED: one block holding the whole row ([S] "Key claims": disabling
//     tiling still fails) -- the shift from all keys, then Ō = bf16(sum P̄ V)
//     with one rounding.
// In fp32-Ō mode nothing is rounded.  Each block takes two passes over its
// keys (scores twice: once for the maximum, once for P̄); the copies are
// synchronous (two barriers a tile).  Tile layout, matrix-instruction
// mapping and masking are those of the streaming kernel.
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ void top2_merge(float& a, float& a2, float b, float b2) {
  float lo = fminf(a, b);
  a = fmaxf(a, b);
  a2 = fmaxf(lo, fmaxf(a2, b2));
}

template <int D, bool CAUSAL, int GUARD, bool OBAR_F32, bool UNTILED>
__global__ __launch_bounds__(kThreads) void fwd_block_kernel(FwdArgs a) {
  // every fp32 operation as written: no multiply is fused into a later add
  // (a fused alpha*R - m would turn r - m = 0 into the rounding error of
  // alpha*R and move decisions taken on it); fused steps are explicit fmaf
#pragma clang fp contract(off)
  constexpr int BN = kFwdBlockN;  // keys per tile
  constexpr int NT = D / kMfmaK;
  constexpr int FB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * D];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int N = a.N;
  const int nmb = (a.N + kFwdBlockM - 1) / kFwdBlockM;
  int head, r;
  xcd_map((int)blockIdx.x, a.B * a.Hq, head, r);
  const int mb = CAUSAL ? (nmb - 1 - r) : r;
  const int hq = head % a.Hq, b = head / a.Hq;
  const int hk = hq / a.group;
  const int q0 = mb * kFwdBlockM + wave * 32;
  const int qrow = q0 + l32;
  const size_t qoff = ((size_t)(b * a.Hq + hq) * N) * D;
  // Ō output and row vectors: dense; Q, K, V, O: the caller's strides
  const uint16_t* __restrict__ Q = a.q + a.lq.head(b, hq);

  // Q fragment as the B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8*half + 0..7]
  bf16x8 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qrow < N) raw = *(const uint4*)(Q + (size_t)qrow * a.lq.sn + 16 * t + 8 * half);
    qf[t] = __builtin_bit_cast(bf16x8, raw);
  }
  f32x16 oacc[FB], bacc[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[f][i] = 0.0f;

  float R = -INFINITY, R2 = -INFINITY;  // running top two of the raw scores
  float m = 0.0f, rt = -INFINITY, lsum = 0.0f;
  bool tie = false;

  const int kend = CAUSAL ? min(N, (mb + 1) * kFwdBlockM) : N;
  const bool wave_live = q0 < N;
  // tiles this wave computes: under the causal mask its rows see no key at
  // or past q0 + 32
  const int wend = !wave_live ? 0 : (CAUSAL ? min(kend, q0 + 32) : kend);
  const i32x4 rk = head_desc(a.k + a.lk.head(b, hk), N, a.lk.sn, D),
             rv = head_desc(a.v + a.lv.head(b, hk), N, a.lv.sn, D);
  const int ksn = a.lk.sn, vsn = a.lv.sn;
  int ka_off[2][NT];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < NT; ++t) ka_off[kb][t] = qidx<D>(32 * kb + l32, 16 * t + 8 * half);
  const int trow = 4 * (g16 >> 1) + (r16 >> 2);
  int ta_off[FB][2];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      ta_off[f][e] = qidx<D>(trow + 8 * e, 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3));

  // S^T = K Q^T for the tile's 64 keys, masked: key of s[kb][i] in this lane
  // is j0 + 32kb + 8(i/4) + 4*half + i%4
  auto scores = [&](int j0, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 kf = *(const bf16x8*)(&Ks[ka_off[kb][t]]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kb], 0, 0, 0);
      }
    }
    if ((j0 + BN > N) || (CAUSAL && j0 + BN - 1 > q0)) {
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - j0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
  };
  // one tile into LDS: every wave is done with the previous one first
  auto load = [&](int j0, bool with_v) {
    __syncthreads();
    dma_tile<D, BN, kWaves>(rk, j0, ksn, wave, lane, Ks);
    if (with_v) dma_tile<D, BN, kWaves>(rv, j0, vsn, wave, lane, Vs);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };

  const int BB = UNTILED ? kend : kFwdOpsBlockN;
  for (int b0 = 0; b0 < kend; b0 += BB) {
    const int b1 = min(b0 + BB, kend);
    // ---- pass 1: running top two over the block's keys
    for (int j0 = b0; j0 < b1; j0 += BN) {
      load(j0, false);
      if (j0 < wend) {
        f32x16 s[2];
        scores(j0, s);
        float tr = -INFINITY, tr2 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float x = s[kb][i], y = s[kb][i + 1];
            tr2 = fmaxf(tr2, __builtin_amdgcn_fmed3f(tr, x, y));
            tr = fmaxf(tr, fmaxf(x, y));
          }
        const auto a1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tr), __float_as_uint(tr), false, false);
        const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tr2), __float_as_uint(tr2), false, false);
        tr = __uint_as_float(a1[0]);
        tr2 = __uint_as_float(a2[0]);
        top2_merge(tr, tr2, __uint_as_float(a1[1]), __uint_as_float(a2[1]));
        top2_merge(R, R2, tr, tr2);
      }
    }
    // ---- the block's decision: tie, shift, rescale of Ō and ℓ
    float m2 = 0.0f;
    if (b0 < wend) {
      rt = a.alpha * R;
      const float r2t = a.alpha * R2;
      tie = (rt - r2t) <= a.tie_eps;
      float mn = rt;
      if (GUARD == kGuardBeta && tie) mn = (rt > 0.0f) ? a.beta * rt : 0.0f;
      if (GUARD == kGuardEps && tie) mn = rt + a.shift_eps;
      const float c = (b0 == 0 || mn == m) ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
      lsum *= c;
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[f][i] *= c;
      m = mn;
      m2 = m * kLog2e;
    }
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) bacc[f][i] = 0.0f;
    // ---- pass 2: P̄, ℓ and the block product B = V^T P̄^T
    for (int j0 = b0; j0 < b1; j0 += BN) {
      load(j0, true);
      if (j0 < wend) {
        f32x16 s[2];
        scores(j0, s);
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], a.c1, -m2));
            lsum += p;
            pf[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
          }
#pragma unroll
        for (int f = 0; f < FB; ++f)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int o0 = ta_off[f][0] + 16 * t * D, o1 = ta_off[f][1] + 16 * t * D;
            const bf16x8 vf = frag2(lds_read_tr(Vs + o0), lds_read_tr(Vs + o1));
            bacc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], bacc[f], 0, 0, 0);
          }
      }
    }
    // ---- block end: Ō = bf16(cŌ + bf16(B)) (bf16 mode) or cŌ + B
    if (b0 < wend) {
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          oacc[f][i] = OBAR_F32 ? oacc[f][i] + bacc[f][i] : bf16_round(oacc[f][i] + bf16_round(bacc[f][i]));
    }
  }

  if (!wave_live) return;
  // ---- epilogue: O = bf16(Ō / ℓ); row outputs
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (qrow >= N) return;
  uint16_t* orow = a.o + a.lo.head(b, hq) + (size_t)qrow * a.lo.sn;
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * f + 8 * g + 4 * half;
      uint16_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = bf16_bits(oacc[f][4 * g + u] / ltot);
      *(uint2*)(orow + col) = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
      if (a.obar) {
        if (OBAR_F32) {
          float* ob = (float*)a.obar + qoff + (size_t)qrow * D + col;
          *(f32x4*)ob = f32x4{oacc[f][4 * g], oacc[f][4 * g + 1], oacc[f][4 * g + 2], oacc[f][4 * g + 3]};
        } else {
          uint16_t* ob = (uint16_t*)a.obar + qoff + (size_t)qrow * D + col;
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = bf16_bits(oacc[f][4 * g + u]);
          *(uint2*)ob = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
        }
      }
    }
  if (half == 0) {
    const size_t ridx = (size_t)(b * a.Hq + hq) * N + qrow;
    a.row_m[ridx] = m;
    a.row_l[ridx] = ltot;
    uint8_t fl = 0;
    if (tie) fl |= 1u;
    if (ltot == 0.0f) fl |= 2u;
    if (tie && GUARD != kGuardNone) fl |= 4u;
    a.row_flags[ridx] = fl;
    if (a.row_max) a.row_max[ridx] = rt;
  }
}

template <int D, bool CAUSAL, int GUARD, bool OBAR_F32>
hipError_t launch_u(const FwdArgs& a, bool untiled, hipStream_t s) {
  const int nmb = (a.N + kFwdBlockM - 1) / kFwdBlockM;
  dim3 grid((unsigned)(nmb * a.Hq * a.B));
  if (untiled)
    hipLaunchKernelGGL((fwd_block_kernel<D, CAUSAL, GUARD, OBAR_F32, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_block_kernel<D, CAUSAL, GUARD, OBAR_F32, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int GUARD>
hipError_t launch_o(const FwdArgs& a, bool obar_f32, bool untiled, hipStream_t s) {
  return obar_f32 ? launch_u<D, CAUSAL, GUARD, true>(a, untiled, s)
                  : launch_u<D, CAUSAL, GUARD, false>(a, untiled, s);
}

template <int D, bool CAUSAL>
hipError_t launch_g(const FwdArgs& a, int guard, bool obar_f32, bool untiled, hipStream_t s) {
  switch (guard) {
    case kGuardBeta: return launch_o<D, CAUSAL, kGuardBeta>(a, obar_f32, untiled, s);
    case kGuardEps: return launch_o<D, CAUSAL, kGuardEps>(a, obar_f32, untiled, s);
    default: return launch_o<D, CAUSAL, kGuardNone>(a, obar_f32, untiled, s);
  }
}

}  // namespace

hipError_t launch_fwd_block(const FwdArgs& a, int d, bool causal, int guard, bool obar_f32,
                            bool untiled, hipStream_t s) {
  if (d == 64)
    return causal ? launch_g<64, true>(a, guard, obar_f32, untiled, s)
                  : launch_g<64, false>(a, guard, obar_f32, untiled, s);
  return causal ? launch_g<128, true>(a, guard, obar_f32, untiled, s)
                : launch_g<128, false>(a, guard, obar_f32, untiled, s);
}

}  // namespace attn
