// attn_bwd.hip -- backward of the guarded streaming attention, gfx950.
//
// What it computes ([R] = the priors.kr review "BF16 플래시 어텐션은 왜 수천
// 스텝 뒤에 무너질까", "Core idea" -> equations, paper Eq. 1-2, and the
// method section, paper §3.2):
//   delta = rowsum(dO∘O) from the bf16 forward output,
//   P     = exp(t - m) / ℓ with the forward's stored (guarded) shift m,
//   dV    = P^T dO,   dP = dO V^T,   dS = P∘(dP - delta),
//   dK    = alpha dS^T Q,   dQ = alpha dS K.
// The guard needs nothing else in the backward: the stored m carries it and
// softmax is unchanged by the shift ([R] the fix, paper §4).
//
// Mapping to CDNA4 (not from the pages):
//   * bwd_pre: one pass over O and dO for delta, and zeroing of the fp32 dQ
//     accumulator;
//   * bwd_main: one workgroup = 4 wave64s = 128 keys of one (batch, KV head);
//     a wave owns 32 keys, keeps their K and V rows in registers and
//     accumulates their dK and dV over every query row (and every query
//     head of the group) in registers -- no atomics for dK/dV;
//   * per step of 32 query rows: Q and dO staged in LDS row-major and
//     transposed; S = Q K^T and dP = dO V^T come out with lane = key and
//     registers = query rows, which is the A-operand layout of dV += P^T dO
//     and dK += dS^T Q, so P and dS go to those products from registers;
//   * dQ needs dS with lane = query row: every wave writes its bf16 dS into
//     one LDS tile, then each wave computes a 16-feature slice of dQ over all
//     128 keys (v_mfma_f32_16x16x32_bf16) and adds it to the fp32
//     accumulator with one atomic per element per workgroup;
//   * bwd_post: dQ = bf16(alpha * accumulator).
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------- bwd_pre
// 8 threads per row (16 bytes each), 32 rows per workgroup.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = 8;            // threads per row
  constexpr int EPT = D / TPR;      // elements per thread (8 or 16)
  const int tid = threadIdx.x;
  const size_t rows = (size_t)a.B * a.Hq * a.N;
  const size_t row = (size_t)blockIdx.x * (kThreads / TPR) + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.0f;
  if (row < rows) {
    const uint16_t* o = a.o + row * D + part * EPT;
    const uint16_t* g = a.dout + row * D + part * EPT;
#pragma unroll
    for (int c = 0; c < EPT; c += 8) {
      const uint4 ov = *(const uint4*)(o + c);
      const uint4 gv = *(const uint4*)(g + c);
      const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(gw[e] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(gw[e] & 0xffff0000u), acc);
      }
    }
    float* dq = a.dq_acc + row * D + part * EPT;
#pragma unroll
    for (int c = 0; c < EPT; c += 4) *(f32x4*)(dq + c) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // reduce over the 8 threads of the row (consecutive lanes)
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------- bwd_post
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_post_kernel(BwdArgs a) {
  const size_t n4 = (size_t)a.B * a.Hq * a.N * D / 4;
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const f32x4 v = *(const f32x4*)(a.dq_acc + 4 * i);
  const uint32_t lo = bf16_bits(a.alpha * v[0]) | ((uint32_t)bf16_bits(a.alpha * v[1]) << 16);
  const uint32_t hi = bf16_bits(a.alpha * v[2]) | ((uint32_t)bf16_bits(a.alpha * v[3]) << 16);
  *(uint2*)(a.dq + 4 * i) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- bwd_main
// Fetch of one 32-row step (Q, dO rows and their statistics) into registers.
template <int D, int CPT>
__device__ __forceinline__ void bwd_fetch(const BwdArgs& a, int sidx, int hk, int b, int qstart,
                                          int nsteps, int tid, uint4 (&qreg)[CPT],
                                          uint4 (&greg)[CPT], float& st_m, float& st_l,
                                          float& st_d) {
  constexpr int BM = kBwdBlockM;
  const int N = a.N;
  const int hq = hk * a.group + sidx / nsteps;
  const int q0 = qstart + (sidx % nsteps) * BM;
  const size_t qoff = ((size_t)(b * a.Hq + hq) * N) * D;
  const size_t roff = (size_t)(b * a.Hq + hq) * N;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    qreg[u] = make_uint4(0, 0, 0, 0);
    greg[u] = make_uint4(0, 0, 0, 0);
    if (q0 + row < N) {
      qreg[u] = *(const uint4*)(a.q + qoff + (size_t)(q0 + row) * D + col);
      greg[u] = *(const uint4*)(a.dout + qoff + (size_t)(q0 + row) * D + col);
    }
  }
  if (tid < BM) {
    const int r = q0 + tid;
    st_m = 0.0f;
    st_l = 0.0f;
    st_d = 0.0f;
    if (r < N) {
      st_m = a.row_m[roff + r] * kLog2e;
      st_l = 1.0f / a.row_l[roff + r];
      st_d = a.delta[roff + r];
    }
  }
}

// Row-major copies, and feature-major copies built from the same registers:
// rows r and r^1 sit in lanes l and l^(D/8); the even row's lane writes
// features col..col+3, the odd row's lane col+4..col+7, one dword (row pair)
// per feature.
template <int D, int CPT, int QSTR, int TSTR>
__device__ __forceinline__ void bwd_stage(int tid, const uint4 (&qreg)[CPT],
                                          const uint4 (&greg)[CPT], float st_m, float st_l,
                                          float st_d, uint16_t* Qs, uint16_t* dOs, uint16_t* Qt,
                                          uint16_t* dOt, float* sm2, float* sinvl, float* sdel) {
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(uint4*)(&Qs[row * QSTR + col]) = qreg[u];
    *(uint4*)(&dOs[row * QSTR + col]) = greg[u];
    const bool even = (row & 1) == 0;
    const int r0 = row & ~1, e0 = even ? 0 : 4;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint4 mine = which ? greg[u] : qreg[u];
      const uint32_t m0 = even ? mine.x : mine.z, m1 = even ? mine.y : mine.w;
      const uint32_t o0 = even ? mine.z : mine.x, o1 = even ? mine.w : mine.y;
      // the partner needs the words this lane does not write
      const uint32_t p0 = (uint32_t)__shfl_xor((int)o0, D / 8);
      const uint32_t p1 = (uint32_t)__shfl_xor((int)o1, D / 8);
      const uint32_t lo0 = even ? m0 : p0, hi0 = even ? p0 : m0;
      const uint32_t lo1 = even ? m1 : p1, hi1 = even ? p1 : m1;
      uint16_t* dst = which ? dOt : Qt;
      *(uint32_t*)(&dst[(col + e0 + 0) * TSTR + r0]) = (lo0 & 0xffffu) | (hi0 << 16);
      *(uint32_t*)(&dst[(col + e0 + 1) * TSTR + r0]) = (lo0 >> 16) | (hi0 & 0xffff0000u);
      *(uint32_t*)(&dst[(col + e0 + 2) * TSTR + r0]) = (lo1 & 0xffffu) | (hi1 << 16);
      *(uint32_t*)(&dst[(col + e0 + 3) * TSTR + r0]) = (lo1 >> 16) | (hi1 & 0xffff0000u);
    }
  }
  if (tid < kBwdBlockM) {
    sm2[tid] = st_m;
    sinvl[tid] = st_l;
    sdel[tid] = st_d;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdArgs a) {
  constexpr int BN = 128;            // keys per workgroup
  constexpr int BM = kBwdBlockM;     // query rows per step (32)
  constexpr int NT = D / kMfmaK;     // 16-wide steps along d
  constexpr int FB = D / 32;         // 32-feature blocks of dK/dV
  constexpr int QSTR = D + 8;        // row stride of the row-major tiles
  constexpr int TSTR = BM + 4;       // row stride of the transposed tiles
  constexpr int SSTR = BN + 8;       // row stride of the dS tile
  constexpr int KTSTR = BN + 8;      // row stride of the transposed K tile
  constexpr int DQB = D / 16 / 4;    // 16-feature dQ slices per wave (1 or 2)

  __shared__ __attribute__((aligned(16))) uint16_t Qs[BM * QSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BM * QSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[BM * SSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * KTSTR];
  __shared__ __attribute__((aligned(16))) float sm2[BM];
  __shared__ __attribute__((aligned(16))) float sinvl[BM];
  __shared__ __attribute__((aligned(16))) float sdel[BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nkb = (N + BN - 1) / BN;
  int kvhead, kblk;
  xcd_map((int)blockIdx.x, nkb, a.B * a.Hkv, kvhead, kblk);
  const int hk = kvhead % a.Hkv, b = kvhead / a.Hkv;
  const int k0 = kblk * BN;
  const int wk0 = k0 + 32 * wave;     // this wave's first key
  const int key = wk0 + l32;          // the key this lane owns in S/dP
  const size_t kvoff = ((size_t)(b * a.Hkv + hk) * N) * D;
  const uint16_t* __restrict__ K = a.k + kvoff;
  const uint16_t* __restrict__ V = a.v + kvoff;

  // K and V rows of this lane's key as B operands: [16t + 8*half + 0..7]
  bf16x8 kf[NT], vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (key < N) {
      kr = *(const uint4*)(K + (size_t)key * D + 16 * t + 8 * half);
      vr = *(const uint4*)(V + (size_t)key * D + 16 * t + 8 * half);
    }
    kf[t] = __builtin_bit_cast(bf16x8, kr);
    vf[t] = __builtin_bit_cast(bf16x8, vr);
  }
  // the workgroup's 128 K rows, feature-major, for the dQ product
  {
    constexpr int CH = (BN / 2) * (D / 8);
    for (int c = tid; c < CH; c += kThreads) {
      const int pr = c % (BN / 2), col = (c / (BN / 2)) * 8;
      const int kk = k0 + 2 * pr;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (kk < N) v0 = *(const uint4*)(K + (size_t)kk * D + col);
      if (kk + 1 < N) v1 = *(const uint4*)(K + (size_t)(kk + 1) * D + col);
      const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *(uint32_t*)(&Kt[(col + 2 * e) * KTSTR + 2 * pr]) = (w0[e] & 0xffffu) | (w1[e] << 16);
        *(uint32_t*)(&Kt[(col + 2 * e + 1) * KTSTR + 2 * pr]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
      }
    }
  }

  f32x16 dk[FB], dv[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[f][i] = 0.0f;
      dv[f][i] = 0.0f;
    }

  // Steps: every 32-row slice of every query head of the group.  The next
  // step's Q, dO and row statistics are fetched into registers while the
  // current step computes; its LDS tiles are written right after the dS
  // barrier of the current step (the staging tiles are free by then).
  const int qstart = CAUSAL ? k0 : 0;  // earlier rows cannot see these keys
  const int nsteps = (N - qstart + BM - 1) / BM;
  const int total = nsteps * a.group;
  constexpr int CH = BM * D / 8;       // 16-byte chunks per tensor per step
  constexpr int CPT = CH / kThreads;   // per thread: 1 (d=64) or 2 (d=128)
  static_assert(CH % kThreads == 0, "step / thread split");
  uint4 qreg[CPT], greg[CPT];
  float st_m = 0.0f, st_l = 0.0f, st_d = 0.0f;

  bwd_fetch<D, CPT>(a, 0, hk, b, qstart, nsteps, tid, qreg, greg, st_m, st_l, st_d);
  bwd_stage<D, CPT, QSTR, TSTR>(tid, qreg, greg, st_m, st_l, st_d, Qs, dOs, Qt, dOt, sm2, sinvl, sdel);
  for (int sidx = 0; sidx < total; ++sidx) {
    const int hq = hk * a.group + sidx / nsteps;
    const int q0 = qstart + (sidx % nsteps) * BM;
    float* __restrict__ dQ = a.dq_acc + ((size_t)(b * a.Hq + hq) * N) * D;
    __syncthreads();  // this step's tiles are visible; the dS tile is free
    if (sidx + 1 < total)
      bwd_fetch<D, CPT>(a, sidx + 1, hk, b, qstart, nsteps, tid, qreg, greg, st_m, st_l, st_d);

    {
      const bool active = wk0 < N && (!CAUSAL || q0 + BM - 1 >= wk0);
      if (active) {
        // ---- S = Q K^T and dP = dO V^T: lane = key, register i = row 8(i/4)+4*half+i%4
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = 0.0f;
          dp[i] = 0.0f;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 qa = *(const bf16x8*)(&Qs[l32 * QSTR + 16 * t + 8 * half]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[t], s, 0, 0, 0);
          const bf16x8 ga = *(const bf16x8*)(&dOs[l32 * QSTR + 16 * t + 8 * half]);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[t], dp, 0, 0, 0);
        }
        // ---- P = exp(t - m)/ℓ and dS = P (dP - delta)
        bf16x8 pa[2], sa[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rl = 8 * g + 4 * half;  // first of the 4 rows of this group
          const f32x4 mv = *(const f32x4*)(&sm2[rl]);
          const f32x4 lv = *(const f32x4*)(&sinvl[rl]);
          const f32x4 dv4 = *(const f32x4*)(&sdel[rl]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * g + u;
            const int qr = q0 + rl + u;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.c1, -mv[u])) * lv[u];
            const bool vis = key < N && qr < N && (!CAUSAL || key <= qr);
            if (!vis) p = 0.0f;
            const float ds = vis ? p * (dp[i] - dv4[u]) : 0.0f;
            pa[i >> 3][i & 7] = (__bf16)p;
            sa[i >> 3][i & 7] = (__bf16)ds;
            dSs[(rl + u) * SSTR + 32 * wave + l32] = bf16_bits(ds);
          }
        }
        // ---- dV += P^T dO and dK += dS^T Q (contraction over the 32 rows,
        // register 8t+j holds row 16t + 8(j/4) + 4*half + j%4)
#pragma unroll
        for (int f = 0; f < FB; ++f) {
          const uint16_t* gr = &dOt[(32 * f + l32) * TSTR];
          const uint16_t* qr = &Qt[(32 * f + l32) * TSTR];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint2 glo = *(const uint2*)(gr + 16 * t + 4 * half);
            const uint2 ghi = *(const uint2*)(gr + 16 * t + 8 + 4 * half);
            const bf16x8 gb = __builtin_bit_cast(bf16x8, make_uint4(glo.x, glo.y, ghi.x, ghi.y));
            dv[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], gb, dv[f], 0, 0, 0);
            const uint2 qlo = *(const uint2*)(qr + 16 * t + 4 * half);
            const uint2 qhi = *(const uint2*)(qr + 16 * t + 8 + 4 * half);
            const bf16x8 qb = __builtin_bit_cast(bf16x8, make_uint4(qlo.x, qlo.y, qhi.x, qhi.y));
            dk[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], qb, dk[f], 0, 0, 0);
          }
        }
      } else {
        // nothing visible: this wave's dS columns are zero
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dSs[(8 * (i >> 2) + 4 * half + (i & 3)) * SSTR + 32 * wave + l32] = 0;
      }
    }
    __syncthreads();  // the dS tile is complete; the staging tiles are free
    if (sidx + 1 < total)
      bwd_stage<D, CPT, QSTR, TSTR>(tid, qreg, greg, st_m, st_l, st_d, Qs, dOs, Qt, dOt, sm2, sinvl, sdel);

    // ---- dQ[q0..q0+31][16-feature slice] += dS K over the 128 keys
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int sl = 0; sl < DQB; ++sl) {
      const int d0 = 16 * (wave * DQB + sl);
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk) {
          const bf16x8 da = *(const bf16x8*)(&dSs[(16 * mq + lr) * SSTR + 32 * kk + 8 * lq]);
          const bf16x8 kb = *(const bf16x8*)(&Kt[(d0 + lr) * KTSTR + 32 * kk + 8 * lq]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, kb, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qr = q0 + 16 * mq + 4 * lq + i;
          if (qr < N) unsafeAtomicAdd(&dQ[(size_t)qr * D + d0 + lr], acc[i]);
        }
      }
    }
  }

  // ---- dK = alpha * sum dS^T Q, dV = sum P^T dO for this wave's 32 keys
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = wk0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (kr < N) {
        const size_t off = kvoff + (size_t)kr * D + 32 * f + l32;
        a.dk[off] = bf16_bits(a.alpha * dk[f][i]);
        a.dv[off] = bf16_bits(dv[f][i]);
      }
    }
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a, int d, hipStream_t s) {
  const size_t rows = (size_t)a.B * a.Hq * a.N;
  const dim3 grid((unsigned)((rows + 31) / 32));
  if (d == 64)
    hipLaunchKernelGGL(bwd_pre_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  const dim3 grid((unsigned)(((a.N + 127) / 128) * a.Hkv * a.B));
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((bwd_main_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_main_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((bwd_main_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_main_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_post(const BwdArgs& a, int d, hipStream_t s) {
  const size_t n4 = (size_t)a.B * a.Hq * a.N * d / 4;
  const dim3 grid((unsigned)((n4 + kThreads - 1) / kThreads));
  if (d == 64)
    hipLaunchKernelGGL(bwd_post_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_post_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
