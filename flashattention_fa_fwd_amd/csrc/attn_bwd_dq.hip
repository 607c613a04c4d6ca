// attn_bwd_dq.hip -- the dQ kernel (which also forms delta) of the guarded
// attention backward, gfx950.
//
// What the backward computes ([R] = the priors.kr review "BF16 플래시 어텐션은
// 왜 수천 스텝 뒤에 무너질까", "Core idea" -> equations, paper Eq. 1-2, and the
// method section, paper §3.2):
//   delta = rowsum(dO∘O) from the bf16 forward output,
//   P     = exp(t - m) / ℓ with the forward's stored (guarded) shift m,
//   dV    = P^T dO,   dP = dO V^T,   dS = P∘(dP - delta),
//   dK    = alpha dS^T Q,   dQ = alpha dS K.
// The guard needs nothing else in the backward: the stored m carries it and
// softmax is unchanged by the shift ([R] the fix, paper §4).
//
// Mapping to CDNA4 (not from the pages): runs first; one workgroup = 128
// query rows, a wave owns 32 of them (lane = row); it forms delta for its
// rows from their O and dO (and writes it for the dK/dV kernel), then
// streams the keys in blocks of 64 like the forward: S^T = K Q^T and dP^T =
// V dO^T, then dS^T in registers is the B operand of dQ^T += K^T dS^T, K^T
// read from the row-major K tile through the transpose read.  dQ is finished
// in registers: no atomics and no fp32 accumulator in memory, and each dQ
// element is written once by one workgroup (bitwise reproducible).
#include "attn_bwd_common.h"

namespace attn {
namespace {

// ---------------------------------------------------------------- bwd_dq
constexpr int kDqRows = 128;  // query rows per workgroup (32 per wave)
constexpr int kDqKeys = 64;   // keys per streaming step

// One streaming step of the dQ kernel for one wave (keys j0..j0+63), after
// the barrier that published the step's K/V tiles: the copy of the next
// tiles first, then S^T, dP^T, dS^T and the dQ^T product.
template <int D, bool CAUSAL, bool DSUM>
__device__ __forceinline__ void dq_step(
    const BwdArgs& a, f32x16 (&dq)[D / 32], float& dsum, const bf16x8 (&qf)[D / kMfmaK],
    const bf16x8 (&gf)[D / kMfmaK], const int (&ka_off)[2][D / kMfmaK], const int (&ta_off)[D / 32][2],
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs,
    uint16_t* __restrict__ ks_next, uint16_t* __restrict__ vs_next, i32x4 rk,
    i32x4 rv, bool more, int j0, int wave, int lane, bool wave_live, int q0,
    int qrow, int half, float lse2, float del) {
  constexpr int BN = kDqKeys;
  constexpr int NT = D / kMfmaK;
  constexpr int FB = D / 32;
  const int N = a.N;
  if (more) {
    dma_tile<D, BN, kWaves>(rk, j0 + BN, a.lk.sn, wave, lane, ks_next);
    dma_tile<D, BN, kWaves>(rv, j0 + BN, a.lv.sn, wave, lane, vs_next);
  }
  // a wave whose rows all lie above this block's first key has nothing here
  if (wave_live && !(CAUSAL && j0 > q0 + 31)) {
    // ---- S^T = K Q^T and dP^T = V dO^T for the 64 keys: lane = row,
    // register i of block kb = key j0 + 32kb + 8(i/4) + 4*half + i%4
    f32x16 sv[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[kb][i] = 0.0f;
        dp[kb][i] = 0.0f;
      }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(&ks[ka_off[kb][t]]);
        sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sv[kb], 0, 0, 0);
        const bf16x8 vf = *(const bf16x8*)(&vs[ka_off[kb][t]]);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[t], dp[kb], 0, 0, 0);
      }
    // ---- dS = P (dP - delta), P = exp2(s * alpha*log2(e) - lse2)
    float dsv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dsv[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][i], a.c1, -lse2)) * (dp[kb][i] - del);
    // only the block holding the diagonal (causal) or the sequence end masks
    const bool edge = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > q0);
    if (__builtin_expect(edge, 0)) {
      asm volatile("");
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - j0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) dsv[kb][i] = 0.0f;
    }
    if constexpr (DSUM) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dsum += dsv[kb][i];
    }
    // dS^T in bf16 as the B operand of dQ^T += K^T dS^T: product t covers
    // keys 16t..16t+15, its k index 8*half + j is key 16t + 8(j/4) +
    // 4*half + j%4, i.e. element i = 8(t%2) + j of block kb = t/2
    bf16x8 sb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float* e = &dsv[t >> 1][8 * (t & 1)];
      sb[t] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]),
                                                    pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7])));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        // keys 16t + trow and 16t + 8 + trow (the swizzle ignores bit 4 and up)
        const int o0 = ta_off[f][0] + 16 * t * D, o1 = ta_off[f][1] + 16 * t * D;
        const bf16x8 kt = frag2(lds_read_tr(ks + o0), lds_read_tr(ks + o1));
        dq[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, sb[t], dq[f], 0, 0, 0);
      }
    }
  }
}

// One streaming step of the first sweep of the dQ kernel in the
// delta = rowsum(dP∘P) mode ([R] method, paper §3.2; [S] "Key claims"):
// S^T and dP^T for the 64 keys as in dq_step, P = exp2(s * alpha*log2(e) -
// lse2), and acc += P dP over the lane's visible keys (in fp32, in key
// order; the other half of the row's keys is in lane ^ 32).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_delta_step(
    const BwdArgs& a, float& acc, const bf16x8 (&qf)[D / kMfmaK], const bf16x8 (&gf)[D / kMfmaK],
    const int (&ka_off)[2][D / kMfmaK], const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, uint16_t* __restrict__ ks_next,
    uint16_t* __restrict__ vs_next, i32x4 rk, i32x4 rv, bool more, int j0, int wave, int lane,
    bool wave_live, int q0, int qrow, int half, float lse2) {
  constexpr int BN = kDqKeys;
  constexpr int NT = D / kMfmaK;
  const int N = a.N;
  if (more) {
    dma_tile<D, BN, kWaves>(rk, j0 + BN, a.lk.sn, wave, lane, ks_next);
    dma_tile<D, BN, kWaves>(rv, j0 + BN, a.lv.sn, wave, lane, vs_next);
  }
  if (wave_live && !(CAUSAL && j0 > q0 + 31)) {
    f32x16 sv[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[kb][i] = 0.0f;
        dp[kb][i] = 0.0f;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 kf = *(const bf16x8*)(&ks[ka_off[kb][t]]);
        sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sv[kb], 0, 0, 0);
        const bf16x8 vf = *(const bf16x8*)(&vs[ka_off[kb][t]]);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[t], dp[kb], 0, 0, 0);
      }
    }
    float pv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pv[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][i], a.c1, -lse2));
    const bool edge = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > q0);
    if (__builtin_expect(edge, 0)) {
      asm volatile("");
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - j0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) pv[kb][i] = 0.0f;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = __builtin_fmaf(pv[kb][i], dp[kb][i], acc);
  }
}

// DELTA_DP: delta = rowsum(dP∘P) from a first sweep over the keys instead
// of rowsum(dO∘O) from the bf16 O.  DSUM: also the row sums of dS (fp32,
// before the bf16 rounding of the dQ operand, without the factor alpha).
template <int D, bool CAUSAL, bool DELTA_DP, bool DSUM>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = kDqKeys;
  constexpr int NT = D / kMfmaK;     // 16-wide steps along d
  constexpr int FB = D / 32;         // 32-feature blocks of dQ
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int N = a.N;
  const int nmb = (N + kDqRows - 1) / kDqRows;
  int head, r;
  xcd_map((int)blockIdx.x, a.B * a.Hq, head, r);
  const int mb = CAUSAL ? (nmb - 1 - r) : r;  // heavy (causal) blocks first
  const int hq = head % a.Hq, b = head / a.Hq;
  const int hk = hq / a.group;
  const int q0 = mb * kDqRows + wave * 32;
  const int qrow = q0 + l32;
  const i32x4 rk = head_desc(a.k + a.lk.head(b, hk), N, a.lk.sn, D);
  const i32x4 rv = head_desc(a.v + a.lv.head(b, hk), N, a.lv.sn, D);
  const uint16_t* __restrict__ Qh = a.q + a.lq.head(b, hq);
  const uint16_t* __restrict__ dOh = a.dout + a.ldo.head(b, hq);

  // Every load of the prologue is issued before the first wait (one memory
  // round trip instead of three): the row's Q and dO fragments (B operands:
  // [16t + 8*half + 0..7]), its O (for delta), m and ℓ, and the first K/V
  // tile.  Rows past the end read the last row; nothing of theirs is stored.
  const int qc = min(qrow, N - 1);
  bf16x8 qf[NT], gf[NT];
  uint4 orw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qf[t] = __builtin_bit_cast(bf16x8, *(const uint4*)(Qh + (size_t)qc * a.lq.sn + 16 * t + 8 * half));
    gf[t] = __builtin_bit_cast(bf16x8, *(const uint4*)(dOh + (size_t)qc * a.ldo.sn + 16 * t + 8 * half));
    if constexpr (!DELTA_DP)
      orw[t] = *(const uint4*)(a.o + a.lo.head(b, hq) + (size_t)qc * a.lo.sn + 16 * t + 8 * half);
  }
  const size_t ridx = (size_t)(b * a.Hq + hq) * N + qc;
  const float mrow = a.row_m[ridx], lrow = a.row_l[ridx];
  dma_tile<D, BN, kWaves>(rk, 0, a.lk.sn, wave, lane, Ks[0]);
  dma_tile<D, BN, kWaves>(rv, 0, a.lv.sn, wave, lane, Vs[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const float lse2 = row_lse2(mrow, lrow);
  // delta = rowsum(dO∘O) of this lane's row: its 32 features here, the
  // other 32 (d = 64) in lane ^ 32 (every lane returns the full sum)
  float del = 0.0f;
  if constexpr (!DELTA_DP) {
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint4 grow = __builtin_bit_cast(uint4, gf[t]);
      const uint32_t ow[4] = {orw[t].x, orw[t].y, orw[t].z, orw[t].w};
      const uint32_t gw[4] = {grow.x, grow.y, grow.z, grow.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = __builtin_fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(gw[e] << 16), part);
        part = __builtin_fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(gw[e] & 0xffff0000u), part);
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    del = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (qrow < N && half == 0) a.delta[(size_t)(b * a.Hq + hq) * N + qrow] = del;
  }

  f32x16 dq[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[f][i] = 0.0f;

  int ka_off[2][NT];  // A operand of S^T / dP^T: key row 32kb + l32, chunk 2t + half
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < NT; ++t) ka_off[kb][t] = qidx<D>(32 * kb + l32, 16 * t + 8 * half);
  const int trow = 4 * (g16 >> 1) + (r16 >> 2);  // transpose reads: key within 16
  int ta_off[FB][2];  // A operand of dQ^T (K^T), product t = 0 (keys trow, trow + 8)
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      ta_off[f][e] = qidx<D>(trow + 8 * e, 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3));

  const int kend = CAUSAL ? min(N, (mb + 1) * kDqRows) : N;
  const bool wave_live = q0 < N;

  if constexpr (DELTA_DP) {
    // first sweep: delta = rowsum(dP∘P) over the keys the row sees (its
    // first tile was copied with the prologue's loads)
    float acc = 0.0f;
    for (int j0 = 0; j0 < kend; j0 += BN) {
      const int cur = (j0 / BN) & 1;
      __syncthreads();
      const bool more = j0 + BN < kend;
      dq_delta_step<D, CAUSAL>(a, acc, qf, gf, ka_off, Ks[cur], Vs[cur], Ks[cur ^ 1], Vs[cur ^ 1],
                               rk, rv, more, j0, wave, lane, wave_live, q0, qrow, half, lse2);
      if (more) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
    del = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (qrow < N && half == 0) a.delta[(size_t)(b * a.Hq + hq) * N + qrow] = del;
    // every wave is done with the last tile before stage 0 is refilled
    __syncthreads();
    dma_tile<D, BN, kWaves>(rk, 0, a.lk.sn, wave, lane, Ks[0]);
    dma_tile<D, BN, kWaves>(rv, 0, a.lv.sn, wave, lane, Vs[0]);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  float dsum = 0.0f;
  for (int j0 = 0; j0 < kend; j0 += BN) {
    const int cur = (j0 / BN) & 1;
    // tile j0 is complete; every wave is done with the previous tile
    __syncthreads();
    const bool more = j0 + BN < kend;
    dq_step<D, CAUSAL, DSUM>(a, dq, dsum, qf, gf, ka_off, ta_off, Ks[cur], Vs[cur], Ks[cur ^ 1],
                             Vs[cur ^ 1], rk, rv, more, j0, wave, lane, wave_live, q0, qrow, half,
                             lse2, del);
    // the copies must land before the next barrier publishes the tile
    if (more) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  if constexpr (DSUM) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
    if (qrow < N && half == 0)
      a.row_dsum[(size_t)(b * a.Hq + hq) * N + qrow] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }

  // ---- dQ = bf16(alpha * dQ): lane = row, register i of block f = feature
  // 32f + 8(i/4) + 4*half + i%4
  if (qrow >= N) return;
  uint16_t* drow = a.dq + a.ldq.head(b, hq) + (size_t)qrow * a.ldq.sn;
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * f + 8 * g + 4 * half;
      *(uint2*)(drow + col) =
          make_uint2(pack_bf16(a.alpha * dq[f][4 * g], a.alpha * dq[f][4 * g + 1]),
                     pack_bf16(a.alpha * dq[f][4 * g + 2], a.alpha * dq[f][4 * g + 3]));
    }
}

}  // namespace

template <bool DELTA_DP, bool DSUM>
hipError_t launch_dq_t(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  const dim3 grid((unsigned)(((a.N + kDqRows - 1) / kDqRows) * a.Hq * a.B));
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<64, true, DELTA_DP, DSUM>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, false, DELTA_DP, DSUM>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<128, true, DELTA_DP, DSUM>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<128, false, DELTA_DP, DSUM>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, bool delta_dp, hipStream_t s) {
  const bool dsum = a.row_dsum != nullptr;
  if (delta_dp)
    return dsum ? launch_dq_t<true, true>(a, d, causal, s) : launch_dq_t<true, false>(a, d, causal, s);
  return dsum ? launch_dq_t<false, true>(a, d, causal, s) : launch_dq_t<false, false>(a, d, causal, s);
}

}  // namespace attn
