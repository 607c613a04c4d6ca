// attn_fwd.hip -- guarded streaming FlashAttention forward for gfx950.
//
// What it computes ([R] = the priors.kr review "BF16 플래시 어텐션은 왜 수천
// 스텝 뒤에 무너질까", [S] = the bud-325 summary "Why Low-Precision
// Transformer Training Fails: An Analysis on Flash Attention"):
//   * tiled attention with an online softmax and an unnormalised output
//     Ō = P̄ V, P̄ = exp(t - m), normalised once at the end ([R] "Why it
//     matters", paper §2.2; "Core idea", equations, paper §3.3.2);
//   * the repeated-maximum guard: a row whose maximum r recurs within
//     tie_eps takes the shift beta*r (r > 0) or 0, or r + shift_eps in the
//     eps variant; other rows take r ([R] the fix, paper §4; [S] "Method",
//     Algorithm 1: one extra step inside the tiling loop);
//   * Ō accumulated in fp32 and rounded to bf16 after every 512 keys (the
//     block size of the analysed code, which keeps P̄V in bf16: [R] "Points
//     to doubt") and after the row's last key, or kept in fp32 throughout
//     ([S] "Key claims" and the QK-Guard abstract: fp32 accumulation repairs
//     it).
//
// Mapping to CDNA4 (not from the pages):
//   * one workgroup = 4 wave64s = 128 query rows of one (batch, head); a
//     wave owns 32 rows;
//   * per step of 64 keys the block's K and V rows are copied row-major into
//     one of two LDS stages by buffer-to-LDS loads (the next block is copied
//     while this one computes; one barrier per step), shared by the 4 waves;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane l of a wave owns query
//     row l%32 and holds 32 of that row's 64 scores (the other 32 sit in lane
//     l^32), so the row max, the top-two merge and the row sum are in-lane
//     plus one exchange between the two lane halves;
//   * P̄ goes to bf16 in registers and is used directly as the B operand of
//     O^T = V^T P̄^T, whose accumulator has the same lane-to-row ownership,
//     so the rescale by exp(m_old - m) is a per-lane scalar; the A operand
//     V^T comes from the row-major V tile through the LDS transpose read.
//
// FP8 variant of the P̄V product (the pages leave open how the bias behaves
// with fewer mantissa bits: [R] "Open questions"): P̄ * 2^k and V are rounded
// to OCP E4M3 (v_cvt_pk_fp8_f32, round to nearest even) and multiplied on
// the scaled 64-product instruction (E4M3 formats, unit scales; operands in
// the bf16 path's key order, the four 16-key groups in sequence); the accumulator
// holds 2^k Ō, exact scaling through every fp32 and bf16 rounding, and the
// scale is taken out at the end.  k is per row and per step: 7 -
// floor((r - m) log2 e), which puts the row's largest P̄ = exp(r - m) in
// [128, 256) -- the top binade below E4M3's 448 -- whatever the shift (the
// beta guard's shift makes that P̄ as small as exp(-(beta-1) r), below E4M3's
// range for a fixed scale); when k changes the accumulator is rescaled by
// the power of two along with exp(m_old - m).  A fixed k = 8 is the other
// option.  ℓ stays the sum of the fp32 P̄.
//
// MXFP4 variant (the other format the pages name there): P̄ and V in E2M1
// elements with one E8M0 scale per block of 32 consecutive keys (keys
// 32h..32h+31 of a 64-key step), 2^(floor(log2 amax) - 2) of the block's
// largest magnitude (v_cvt_scalef32_pk_fp4_f32 gives RNE(clamp(v / scale)),
// measured), on v_mfma_scale_f32_32x32x64_f8f6f4: one instruction per
// feature block and 64-key step, whose k index 32h + j is key 32h + j and
// sits in lane half h.  S^T leaves each lane half with every fourth group
// of four keys of both blocks, so one swap of lane halves (permlane32_swap)
// gives half h the 32 P̄ of block h; V^T is read key-block by key-block.
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Four bf16 values (two per word, low half first) to four E4M3 bytes in the
// same order: bf16 -> fp32 is exact, the conversion rounds to nearest even.
__device__ __forceinline__ uint32_t fp8x4_from_bf16x4(uint2 w) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u), r, true);
  return (uint32_t)r;
}

// 2^e as a float for -126 <= e <= 127 (built from the exponent field).
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((127 + e) << 23); }

// Top-two merge of (a, a2) and (b, b2), each with first >= second; the
// result keeps multiset semantics (equal maxima give r2 == r).
__device__ __forceinline__ void top2_merge(float& a, float& a2, float b, float b2) {
  float lo = fminf(a, b);
  a = fmaxf(a, b);
  a2 = fmaxf(lo, fmaxf(a2, b2));
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The matrix operands of Ō's product.
constexpr int kPvBf16 = 0, kPvFp8 = 1, kPvMx = 2;

// Four E2M1 pairs of v / scale (rounded to nearest even, saturating) in
// the four bytes of a word, low byte first.
__device__ __forceinline__ uint32_t fp4x8(const float* v, float scale) {
  uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], scale, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2], v[3], scale, 1);
  uint32_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[4], v[5], scale, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[6], v[7], scale, 1);
  return (lo & 0xffffu) | (hi << 16);
}

// E8M0 byte of the MX scale of a block whose largest magnitude is amax:
// 2^(floor(log2 amax) - 2) from the exponent field (at least 1), or with
// ceil (amax / X in (2, 4]: never saturates) one more unless amax is a
// power of two.
__device__ __forceinline__ int mx_scale_byte(float amax, bool ceil) {
  const uint32_t b = __float_as_uint(amax);
  const int up = (ceil && (b & 0x7fffffu) != 0u) ? 1 : 0;
  return max((int)((b >> 23) & 0xffu) - 2 + up, 1);
}

template <int D, bool CAUSAL, int GUARD, bool OBAR_F32, int PV>
__global__ __launch_bounds__(kThreads, D == 64 ? (PV == 0 ? 4 : 3) : 2) void fwd_kernel(FwdArgs a) {
  // every fp32 operation as written: no multiply is fused into a later add
  // (a fused alpha*R - m would turn r - m = 0 into the rounding error of
  // alpha*R and move decisions taken on it); fused steps are explicit fmaf
#pragma clang fp contract(off)
  constexpr bool PV_FP8 = PV == kPvFp8;
  constexpr bool PV_MX = PV == kPvMx;
  constexpr int BN = kFwdBlockN;
  constexpr int NT = D / kMfmaK; // matrix steps along d for S
  constexpr int FB = D / 32;     // 32-feature blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];
  // FP8 product: the step's V^T operand in E4M3, in operand order ([16-key
  // group t][feature block f][lane], 8 keys a lane); wave w converts group w
  __shared__ __attribute__((aligned(16))) uint2 Vf8[PV == kPvFp8 ? 4 * (D / 32) * 64 : 1];
  // MXFP4 product: the step's V^T operand (E2M1 elements of the lane's 32
  // keys, [feature block f][lane]) and its E8M0 scale bytes; wave w converts
  // the feature blocks f = w, w + 4, ...
  __shared__ __attribute__((aligned(16))) uint4 Vmx[PV == kPvMx ? (D / 32) * 64 : 1];
  __shared__ __attribute__((aligned(16))) int Smx[PV == kPvMx ? (D / 32) * 64 : 1];

  const int tid = threadIdx.x;
  // the wave index is uniform over the wave: keeping it scalar makes every
  // per-wave condition below a scalar branch instead of an exec mask
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int N = a.N;
  const int nmb = (a.N + kFwdBlockM - 1) / kFwdBlockM;
  int head, r;
  xcd_map((int)blockIdx.x, a.B * a.Hq, head, r);
  const int mb = CAUSAL ? (nmb - 1 - r) : r;  // heavy (causal) blocks first
  const int hq = head % a.Hq, b = head / a.Hq;
  const int hk = hq / a.group;
  const int q0 = mb * kFwdBlockM + wave * 32;
  const int qrow = q0 + l32;

  const size_t qoff = ((size_t)(b * a.Hq + hq) * N) * D;
  // Ō output and row vectors: dense; Q, K, V, O: the caller's strides
  const uint16_t* __restrict__ Q = a.q + a.lq.head(b, hq);

  // Q fragment as the B operand: lane holds Q[qrow][16t + 8*half + 0..7]
  bf16x8 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qrow < N) raw = *(const uint4*)(Q + (size_t)qrow * a.lq.sn + 16 * t + 8 * half);
    qf[t] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 oacc[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[f][i] = 0.0f;

  float R = -INFINITY, R2 = -INFINITY;  // running top two of the raw scores s
  float m = 0.0f, m2 = 0.0f, rt = -INFINITY;
  float lsum = 0.0f;
  bool tie = false;
  int pk = 8;  // FP8 product: exponent of the operand scale 2^k

  const int kend = CAUSAL ? min(N, (mb + 1) * kFwdBlockM) : N;
  const bool wave_live = q0 < N;

  const i32x4 rk = head_desc(a.k + a.lk.head(b, hk), N, a.lk.sn, D),
             rv = head_desc(a.v + a.lv.head(b, hk), N, a.lv.sn, D);
  const int ksn = a.lk.sn, vsn = a.lv.sn;
  // per-lane LDS offsets: K rows as the A operand of S^T (key row 32kb + l32,
  // chunk 2t + half); V^T as the A operand of O^T through the transpose read
  // (keys 16t + trow and 16t + 8 + trow, features 32f + 16(g16&1) + ...)
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

  // Steps this wave computes: under the causal mask a wave's rows see no key
  // at or past q0 + 32.  Every wave still takes part in the copies and
  // barriers of the workgroup's remaining steps (second loop below); keeping
  // those in a loop of their own lets the accumulators stay in one register
  // set across the computing steps.
  const int jc = !wave_live ? 0 : (CAUSAL ? min(kend, q0 + 32) : kend);

  // MXFP4 product: this wave's feature blocks of the step's V^T operand,
  // quantized (per lane: one feature, the 32 consecutive keys of its half's
  // block) into LDS
  auto convert_mx = [&](const uint16_t* vs) {
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      if (f % kWaves != wave) continue;  // uniform: static register indices below
      // V^T in key order: vx[o] = V[32*half + o][32f + l32]; transpose read
      // t returns keys 32*half + 4t + 0..3
      float vx[32];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint2 w = lds_read_tr(vs + qidx<D>(32 * half + 4 * t + (r16 >> 2), 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3)));
        vx[4 * t] = __uint_as_float(w.x << 16);
        vx[4 * t + 1] = __uint_as_float(w.x & 0xffff0000u);
        vx[4 * t + 2] = __uint_as_float(w.y << 16);
        vx[4 * t + 3] = __uint_as_float(w.y & 0xffff0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; j += 2) amax = fmaxf(amax, fmaxf(fabsf(vx[j]), fabsf(vx[j + 1])));
      const int sbv = mx_scale_byte(amax, a.pv_mx_ceil != 0);
      const float xs = __int_as_float(sbv << 23);
      Vmx[f * 64 + lane] = make_uint4(fp4x8(&vx[0], xs), fp4x8(&vx[8], xs), fp4x8(&vx[16], xs), fp4x8(&vx[24], xs));
      Smx[f * 64 + lane] = sbv;
    }
  };
  // FP8 product: this wave's share (keys 16*wave .. 16*wave + 15) of the
  // step's E4M3 V^T operand, written for every wave to read after a barrier
  auto convert_v = [&](const uint16_t* vs) {
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int o0 = ta_off[f][0] + 16 * wave * D, o1 = ta_off[f][1] + 16 * wave * D;
      const uint2 v0 = lds_read_tr(vs + o0), v1 = lds_read_tr(vs + o1);
      Vf8[(wave * FB + f) * 64 + lane] = make_uint2(fp8x4_from_bf16x4(v0), fp8x4_from_bf16x4(v1));
    }
  };

  dma_tile<D, BN, kWaves>(rk, 0, ksn, wave, lane, Ks[0]);
  dma_tile<D, BN, kWaves>(rv, 0, vsn, wave, lane, Vs[0]);
  int j0 = 0;
  for (; j0 < jc; j0 += BN) {
    const int cur = (j0 / BN) & 1;
    // this wave's copies of tile j0 have landed (a no-op when none are in
    // flight); after the barrier the whole tile is, and every wave is done
    // with the previous tile
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const bool more = j0 + BN < kend;
    if (more) {
      dma_tile<D, BN, kWaves>(rk, j0 + BN, ksn, wave, lane, Ks[cur ^ 1]);
      dma_tile<D, BN, kWaves>(rv, j0 + BN, vsn, wave, lane, Vs[cur ^ 1]);
    }
    const uint16_t* ks = Ks[cur];
    const uint16_t* vs = Vs[cur];

    // ---- S^T = K Q^T for the 64 keys: two 32-key blocks
    // (the two blocks' chains interleaved: consecutive products are
    // independent)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(&ks[ka_off[kb][t]]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kb], 0, 0, 0);
      }
    if constexpr (PV_FP8) convert_v(vs);
    if constexpr (PV_MX) convert_mx(vs);
    // key of s[kb][i] in this lane: j0 + 32kb + 8(i/4) + 4*half + i%4; only
    // the block holding the diagonal (causal) or the sequence end masks
    const bool edge = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > q0);
    if (__builtin_expect(edge, 0)) {
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - j0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }

    // ---- running top two (repeated-maximum detection), two scores at a
    // time: with tr >= tr2, the second largest of {tr, tr2, x, y} is
    // max(tr2, med3(tr, x, y)) and the largest is max(tr, x, y)
    float tr = -INFINITY, tr2 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float x = s[kb][i], y = s[kb][i + 1];
        tr2 = fmaxf(tr2, __builtin_amdgcn_fmed3f(tr, x, y));
        tr = fmaxf(tr, fmaxf(x, y));
      }
    // merge with the other lane half (same rows): after the swap each lane
    // holds both halves' values, paired by source lane
    {
      const auto a1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tr), __float_as_uint(tr), false, false);
      const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tr2), __float_as_uint(tr2), false, false);
      tr = __uint_as_float(a1[0]);
      tr2 = __uint_as_float(a2[0]);
      top2_merge(tr, tr2, __uint_as_float(a1[1]), __uint_as_float(a2[1]));
    }
    top2_merge(R, R2, tr, tr2);

    // ---- tie decision and shift on the scaled logits t = alpha * s
    rt = a.alpha * R;
    const float r2t = a.alpha * R2;
    tie = (rt - r2t) <= a.tie_eps;  // false when r2 is -inf (a single key)
    float mn = rt;
    if (GUARD == kGuardBeta && tie) mn = (rt > 0.0f) ? a.beta * rt : 0.0f;
    if (GUARD == kGuardEps && tie) mn = rt + a.shift_eps;

    // ---- rescale by c = exp(m_old - m_new); c = 1 exactly where the shift
    // did not move (and on the first step), so multiplying by it changes
    // nothing there and keeps the accumulator in one register set.
    // FP8 product: the operand scale 2^k for this step (r - m <= 0 under
    // every guard, so k >= 7), the accumulator moved to it exactly
    {
      const float c = (j0 == 0 || mn == m) ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
      lsum *= c;
      float co = c;
      if (PV_FP8) {
        int kn = 8;
        if (!a.pv_fixed_scale) kn = 7 - (int)fmaxf(floorf((rt - mn) * kLog2e), -113.0f);
        co = c * pow2i(kn - pk);  // exact: a power of two
        pk = kn;
      }
      // a step that moves no shift of the wave's rows skips the products
      // (x * 1 = x exactly, denormals included)
      if (__builtin_amdgcn_ballot_w64(co != 1.0f) != 0) {
#pragma unroll
        for (int f = 0; f < FB; ++f)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[f][i] *= co;
      }
      m = mn;
    }
    const float psc = PV_FP8 ? pow2i(pk) : 1.0f;
    m2 = m * kLog2e;

    // ---- P̄ = exp(t - m) = exp2(s * alpha*log2e - m*log2e); row sum; the
    // matrix operand in bf16, or 2^k P̄ in E4M3
    bf16x8 pf[4];
    uint32_t pf8[4][2];
    float pmx[32];  // MXFP4: the lane's P̄ in k order 16kb + i
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], a.c1, -m2));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], a.c1, -m2));
        lsum += p0;
        lsum += p1;
        const int t = 2 * kb + (i >> 3), u = i & 7;
        if (PV_FP8) {
          uint32_t& w = pf8[t][u >> 2];
          if (u & 2)
            w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p0 * psc, p1 * psc, (int)w, true);
          else
            w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p0 * psc, p1 * psc, 0, false);
        } else if (PV_MX) {
          pmx[16 * kb + i] = p0;
          pmx[16 * kb + i + 1] = p1;
        } else {
          pf[t][u] = (__bf16)p0;
          pf[t][u + 1] = (__bf16)p1;
        }
      }
    // MXFP4: one block of 32 P̄ per lane, its row's keys 32*half..+31 in
    // key order.  pmx[i] and pmx[16 + i] hold keys 8(i/4) + 4*half + i%4 of
    // block 0 and block 1; after the swap of lane halves w[0] and w[1] hold
    // keys 8(i/4) + i%4 and 8(i/4) + 4 + i%4 of block `half`
    int sbp = 1;
    i32x8 pmb = {0, 0, 0, 0, 0, 0, 0, 0};
    if (PV_MX) {
      float blk[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(pmx[i]), __float_as_uint(pmx[16 + i]), false, false);
        const int o = 8 * (i >> 2) + (i & 3);
        blk[o] = __uint_as_float(w[0]);
        blk[o + 4] = __uint_as_float(w[1]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; j += 2) amax = fmaxf(amax, fmaxf(blk[j], blk[j + 1]));
      sbp = mx_scale_byte(amax, a.pv_mx_ceil != 0);
      const float xs = __int_as_float(sbp << 23);
#pragma unroll
      for (int w = 0; w < 4; ++w) pmb[w] = (int)fp4x8(&blk[8 * w], xs);
    }

    // ---- O^T += V^T P̄^T: four steps of 16 keys, in key order (the feature
    // blocks' chains interleaved); MXFP4: one step of 64 keys
    // every wave's share of the low-precision V^T operand is in LDS
    if constexpr (PV_FP8 || PV_MX) __syncthreads();
    if (PV_FP8) {
      // one scaled 64-product instruction per feature block (E4M3 operands,
      // unit scales): the operand tile holds the four 16-key fragments of a
      // block in sequence and P̄ is packed in the same key order
      const i32x8 pb = {(int)pf8[0][0], (int)pf8[0][1], (int)pf8[1][0], (int)pf8[1][1],
                        (int)pf8[2][0], (int)pf8[2][1], (int)pf8[3][0], (int)pf8[3][1]};
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        const uint2 w0 = Vf8[(0 * FB + f) * 64 + lane], w1 = Vf8[(1 * FB + f) * 64 + lane];
        const uint2 w2 = Vf8[(2 * FB + f) * 64 + lane], w3 = Vf8[(3 * FB + f) * 64 + lane];
        const i32x8 va = {(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y, (int)w2.x, (int)w2.y, (int)w3.x, (int)w3.y};
        // formats 0, 0: E4M3 operands; scale bytes 127 = 2^0
        oacc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, oacc[f], 0, 0, 0, 127, 0, 127);
      }
    }
    if (PV_MX) {
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        const uint4 w = Vmx[f * 64 + lane];
        const int sbv = Smx[f * 64 + lane];
        const i32x8 va = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        // formats 4, 4: E2M1 operands; scale bytes in bits 0..7
        oacc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pmb, oacc[f], 4, 4, 0, sbv, 0, sbp);
      }
    }
#pragma unroll
    for (int t = 0; t < (PV_MX || PV_FP8 ? 0 : 4); ++t) {
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        // A = V^T: feature 32f + l32, keys 16t + 4*half + 0..3 and 16t + 8 + 4*half + 0..3
        const int o0 = ta_off[f][0] + 16 * t * D, o1 = ta_off[f][1] + 16 * t * D;
        const uint2 v0 = lds_read_tr(vs + o0), v1 = lds_read_tr(vs + o1);
        oacc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag2(v0, v1), pf[t], oacc[f], 0, 0, 0);
      }
    }
    // bf16 mode: round the accumulator after every kFwdRoundN keys and
    // after this wave's last step (which holds the last key of its rows)
    const bool last = CAUSAL ? (j0 + BN > q0 + 31) : (j0 + BN >= kend);
    if (!OBAR_F32 && (((j0 + BN) % kFwdRoundN) == 0 || last)) {
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[f][i] = bf16_round(oacc[f][i]);
    }
  }
  for (; j0 < kend; j0 += BN) {
    const int cur = (j0 / BN) & 1;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (j0 + BN < kend) {
      dma_tile<D, BN, kWaves>(rk, j0 + BN, ksn, wave, lane, Ks[cur ^ 1]);
      dma_tile<D, BN, kWaves>(rv, j0 + BN, vsn, wave, lane, Vs[cur ^ 1]);
    }
    // low-precision products: the waves still computing need this wave's share
    if constexpr (PV_FP8) convert_v(Vs[cur]);
    if constexpr (PV_MX) convert_mx(Vs[cur]);
    if constexpr (PV_FP8 || PV_MX) __syncthreads();
  }
  // no copy may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if (!wave_live) return;
  // ---- epilogue: O = bf16(Ō / ℓ); row outputs
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (qrow >= N) return;
  if (PV_FP8) {
    const float un = pow2i(-pk);  // exact
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[f][i] *= un;
  }
  // Ō/ℓ: a reciprocal refined by one Newton step, the product corrected by
  // its exact residual (fma).  For ℓ in [2^-100, 2^100] this equals the
  // IEEE quotient on every pair probed (all 2^23 significands of ℓ at four
  // exponents, five numerators each) at a third of the instructions; a wave
  // holding any other ℓ (0, overflowed) takes the IEEE division.
  float quo[FB][16];
  {
    const bool lnorm = ltot >= 0x1p-100f && ltot <= 0x1p100f;
    if (__all(lnorm)) {
      const float r0 = __builtin_amdgcn_rcpf(ltot);
      const float rl = __builtin_fmaf(__builtin_fmaf(-ltot, r0, 1.0f), r0, r0);
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float q0 = oacc[f][i] * rl;
          quo[f][i] = __builtin_fmaf(__builtin_fmaf(-q0, ltot, oacc[f][i]), rl, q0);
        }
    } else {
      // keep this a branch: selecting between both forms would run both
      asm volatile("");
#pragma unroll
      for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) quo[f][i] = oacc[f][i] / ltot;
    }
  }
  uint16_t* orow = a.o + a.lo.head(b, hq) + (size_t)qrow * a.lo.sn;
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * f + 8 * g + 4 * half;
      uint16_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = bf16_bits(quo[f][4 * g + u]);
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

template <int D, bool CAUSAL, int GUARD, bool OBAR_F32, int PV>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  const int nmb = (a.N + kFwdBlockM - 1) / kFwdBlockM;
  dim3 grid((unsigned)(nmb * a.Hq * a.B));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, GUARD, OBAR_F32, PV>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int GUARD, int PV>
hipError_t launch_o(const FwdArgs& a, bool obar_f32, hipStream_t s) {
  return obar_f32 ? launch_t<D, CAUSAL, GUARD, true, PV>(a, s)
                  : launch_t<D, CAUSAL, GUARD, false, PV>(a, s);
}

template <int D, bool CAUSAL, int PV>
hipError_t launch_g(const FwdArgs& a, int guard, bool obar_f32, hipStream_t s) {
  switch (guard) {
    case kGuardBeta: return launch_o<D, CAUSAL, kGuardBeta, PV>(a, obar_f32, s);
    case kGuardEps: return launch_o<D, CAUSAL, kGuardEps, PV>(a, obar_f32, s);
    default: return launch_o<D, CAUSAL, kGuardNone, PV>(a, obar_f32, s);
  }
}

template <int PV>
hipError_t launch_d(const FwdArgs& a, int d, bool causal, int guard, bool obar_f32, hipStream_t s) {
  if (d == 64)
    return causal ? launch_g<64, true, PV>(a, guard, obar_f32, s)
                  : launch_g<64, false, PV>(a, guard, obar_f32, s);
  return causal ? launch_g<128, true, PV>(a, guard, obar_f32, s)
                : launch_g<128, false, PV>(a, guard, obar_f32, s);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int guard, bool obar_f32, int pv,
                      hipStream_t s) {
  switch (pv) {
    case 1: return launch_d<kPvFp8>(a, d, causal, guard, obar_f32, s);
    case 2: return launch_d<kPvMx>(a, d, causal, guard, obar_f32, s);
    default: return launch_d<kPvBf16>(a, d, causal, guard, obar_f32, s);
  }
}

}  // namespace attn
