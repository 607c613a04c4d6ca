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
  const int kblk = blockIdx.x;
  const int hk = blockIdx.y, b = blockIdx.z;
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

  const int qstart = CAUSAL ? k0 : 0;  // earlier rows cannot see these keys
  for (int hh = 0; hh < a.group; ++hh) {
    const int hq = hk * a.group + hh;
    const size_t qoff = ((size_t)(b * a.Hq + hq) * N) * D;
    const size_t roff = (size_t)(b * a.Hq + hq) * N;
    const uint16_t* __restrict__ Q = a.q + qoff;
    const uint16_t* __restrict__ dO = a.dout + qoff;
    float* __restrict__ dQ = a.dq_acc + qoff;

    for (int q0 = qstart; q0 < N; q0 += BM) {
      __syncthreads();  // everyone is done with the previous step's tiles
      // ---- stage Q and dO rows q0..q0+31: row-major and feature-major
      {
        constexpr int CH = BM * D / 8;  // 16-byte chunks per tensor
        for (int c = tid; c < 2 * CH; c += kThreads) {
          const int which = c / CH, cc = c % CH;
          const int row = cc / (D / 8), col = (cc % (D / 8)) * 8;
          const uint16_t* src = which ? dO : Q;
          uint4 val = make_uint4(0, 0, 0, 0);
          if (q0 + row < N) val = *(const uint4*)(src + (size_t)(q0 + row) * D + col);
          *(uint4*)(&(which ? dOs : Qs)[row * QSTR + col]) = val;
        }
        constexpr int TCH = (BM / 2) * (D / 8);
        for (int c = tid; c < 2 * TCH; c += kThreads) {
          const int which = c / TCH, cc = c % TCH;
          const int pr = cc % (BM / 2), col = (cc / (BM / 2)) * 8;
          const int r = q0 + 2 * pr;
          const uint16_t* src = which ? dO : Q;
          uint16_t* dst = which ? dOt : Qt;
          uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
          if (r < N) v0 = *(const uint4*)(src + (size_t)r * D + col);
          if (r + 1 < N) v1 = *(const uint4*)(src + (size_t)(r + 1) * D + col);
          const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
          const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            *(uint32_t*)(&dst[(col + 2 * e) * TSTR + 2 * pr]) = (w0[e] & 0xffffu) | (w1[e] << 16);
            *(uint32_t*)(&dst[(col + 2 * e + 1) * TSTR + 2 * pr]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
          }
        }
        if (tid < BM) {
          const int r = q0 + tid;
          float mm = 0.0f, il = 0.0f, de = 0.0f;
          if (r < N) {
            mm = a.row_m[roff + r] * kLog2e;
            il = 1.0f / a.row_l[roff + r];
            de = a.delta[roff + r];
          }
          sm2[tid] = mm;
          sinvl[tid] = il;
          sdel[tid] = de;
        }
      }
      __syncthreads();

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
      __syncthreads();

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
  const dim3 grid((unsigned)((a.N + 127) / 128), a.Hkv, a.B);
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
