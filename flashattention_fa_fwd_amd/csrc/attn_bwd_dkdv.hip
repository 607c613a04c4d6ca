// attn_bwd_dkdv.hip -- the dK/dV kernel of the guarded attention backward,
// gfx950.
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
// Mapping to CDNA4 (not from the pages): one workgroup = 4 wave64s = 128
// keys of one (batch, KV head); a wave owns 32 keys and accumulates their dK
// and dV over every query row (and every query head of the group) in
// registers.  Per step of 32 query rows, Q and dO are copied row-major into
// one of two LDS stages by buffer-to-LDS loads (one barrier per step).  S =
// Q K^T and dP = dO V^T come out with lane = key and registers = query rows,
// the A-operand layout of dV += P^T dO and dK += dS^T Q, whose B operands (dO
// and Q, contraction over rows) come from the row-major stages through the
// gfx950 LDS transpose read.  Runs after the dQ kernel, which writes delta.
// dK and dV are each written once by one workgroup (bitwise reproducible).
//
// This translation unit is built with the iterative-ILP instruction
// scheduler (build_lib.py): same instructions and results, 4-9 % less time
// for this kernel in A/B runs.
#include "attn_bwd_common.h"

namespace attn {
namespace {

// ---------------------------------------------------------------- bwd_dkdv
constexpr int kDkdvKeys = 128;  // keys per workgroup (32 per wave)

// Position of a step: query head (within the group) and first row.
struct StepPos {
  int h, q0;
  __device__ __forceinline__ void next(int qstart, int N) {
    q0 += kBwdBlockM;
    if (q0 >= N) {
      q0 = qstart;
      ++h;
    }
  }
};

// Copy one step (Q and dO rows of query head hq, rows q0..q0+31) into a
// stage; threads 0..31 also load the rows' statistics (raw: they are used
// once the copies have landed).
template <int D>
__device__ __forceinline__ void dkdv_load(const BwdArgs& a, int hq, int q0, int b, int wave,
                                          int lane, int tid, uint16_t* Qs, uint16_t* dOs,
                                          float (&stat)[3]) {
  // the copies first: issued after the statistics' loads, their address
  // arithmetic can be given a register that one of those loads is still
  // filling and then waits for it (wave 0 stalled on that every step;
  // 5 % of the kernel at GPT-2 Small)
  dma_tile<D, kBwdBlockM, kWaves>(head_desc(a.q + a.lq.head(b, hq), a.N, a.lq.sn, D), q0, a.lq.sn,
                                  wave, lane, Qs);
  dma_tile<D, kBwdBlockM, kWaves>(head_desc(a.dout + a.ldo.head(b, hq), a.N, a.ldo.sn, D), q0,
                                  a.ldo.sn, wave, lane, dOs);
  // rows past the end read the last row; bwd_stats_store neutralises them
  if (tid < kBwdBlockM) {
    const size_t r = (size_t)(b * a.Hq + hq) * a.N + min(q0 + tid, a.N - 1);
    stat[0] = a.row_m[r];
    stat[1] = a.row_l[r];
    stat[2] = a.delta[r];
  }
}

// Write a step's row statistics to its stage (threads 0..31, rows q0 + tid).
__device__ __forceinline__ void bwd_stats_store(const float (&stat)[3], int q0, int tid, int N,
                                                float* slse, float* sdel) {
  const bool in = q0 + tid < N;
  slse[tid] = in ? row_lse2(stat[0], stat[1]) : 0.0f;
  sdel[tid] = in ? stat[2] : 0.0f;
}

// One step of the dK/dV kernel for one wave, after the barrier that
// published the step's stage: first the copy of the next step into the
// other stage, then S, dP, P, dS and the dV/dK products.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_step(
    const BwdArgs& a, f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const int (&qa_off)[D / kMfmaK],
    const int (&ka_off)[D / kMfmaK], const int (&tb_off)[D / 32][2], const uint16_t* __restrict__ qs,
    const uint16_t* __restrict__ gs, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, const bf16x8 (&vfr)[D / kMfmaK], const float* __restrict__ slse,
    const float* __restrict__ sdel, uint16_t* __restrict__ qs_next,
    uint16_t* __restrict__ gs_next, bool more, int hq_next, int q0_next, int b, int wave,
    int lane, int tid, float (&stat)[3], int q0, int wk0, int key, int half) {
  constexpr int BM = kBwdBlockM;
  constexpr int NT = D / kMfmaK;
  constexpr int FB = D / 32;
  const int N = a.N;
  if (more) dkdv_load<D>(a, hq_next, q0_next, b, wave, lane, tid, qs_next, gs_next, stat);
  const bool live = wk0 < N && (!CAUSAL || q0 + BM - 1 >= wk0);
  if (live) {
    // ---- S = Q K^T and dP = dO V^T: lane = key, register i = row 8(i/4)+4*half+i%4
    f32x16 sv, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = 0.0f;
      dp[i] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 kb = *(const bf16x8*)(&ks[ka_off[t]]);
      const bf16x8 qa = *(const bf16x8*)(&qs[qa_off[t]]);
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, sv, 0, 0, 0);
      bf16x8 vb;
      if constexpr (D == 128)
        vb = vfr[t];
      else
        vb = *(const bf16x8*)(&vs[ka_off[t]]);
      const bf16x8 ga = *(const bf16x8*)(&gs[qa_off[t]]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vb, dp, 0, 0, 0);
    }
    // ---- P = exp2(s * alpha*log2(e) - lse2) and dS = P (dP - delta)
    float pv[16], dsv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rl = 8 * g + 4 * half;  // first of the 4 rows of this group
      const f32x4 lv = *(const f32x4*)(&slse[rl]);
      const f32x4 dl = *(const f32x4*)(&sdel[rl]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 4 * g + u;
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], a.c1, -lv[u]));
        dsv[i] = pv[i] * (dp[i] - dl[u]);
      }
    }
    // only the block on the diagonal and the ragged ends mask: element i
    // (row q0 + 4*half + r_i, r_i = 8(i/4) + i%4) is visible iff
    // lo <= r_i < hi
    const bool edge = (CAUSAL && wk0 + 31 > q0) || q0 + BM > N || wk0 + 32 > N;
    if (__builtin_expect(edge, 0)) {
      // an empty volatile asm keeps this block a branch: the compiler
      // would otherwise turn it into selects executed on every step
      asm volatile("");
      const int lo = CAUSAL ? key - q0 - 4 * half : 0;
      const int hi = key < N ? N - q0 - 4 * half : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ri = 8 * (i >> 2) + (i & 3);
        if (ri < lo || ri >= hi) {
          pv[i] = 0.0f;
          dsv[i] = 0.0f;
        }
      }
    }
    // bf16 operands: register 8t+j of pa/sa is element i = 8t+j
    bf16x8 pa[2], sa[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float* p = &pv[8 * t];
      const float* d = &dsv[8 * t];
      pa[t] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                                    pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])));
      sa[t] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(d[0], d[1]), pack_bf16(d[2], d[3]),
                                                    pack_bf16(d[4], d[5]), pack_bf16(d[6], d[7])));
    }
    // ---- dV += P^T dO and dK += dS^T Q, contraction over the 32 rows:
    // the k index 8*half + j of product t is row 16t + 8(j/4) + 4*half +
    // j%4, so the B operand is two transpose reads of 4 rows each
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        // rows 16t + trow and 16t + 8 + trow (the swizzle ignores bit 4 and up)
        const int o0 = tb_off[f][0] + 16 * t * D, o1 = tb_off[f][1] + 16 * t * D;
        const bf16x8 gb = frag2(lds_read_tr(gs + o0), lds_read_tr(gs + o1));
        dv[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], gb, dv[f], 0, 0, 0);
        const bf16x8 qb = frag2(lds_read_tr(qs + o0), lds_read_tr(qs + o1));
        dk[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], qb, dk[f], 0, 0, 0);
      }
    }
  }
}

// d = 64: three workgroups per CU (at most 168 VGPRs a wave); d = 128 needs
// more registers.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BN = kDkdvKeys;
  constexpr int BM = kBwdBlockM;     // query rows per step (32)
  constexpr int NT = D / kMfmaK;     // 16-wide steps along d
  constexpr int FB = D / 32;         // 32-feature blocks of dK/dV

  // two stages: step s computes from stage s&1 while step s+1 is copied
  // into the other
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * D];
  __shared__ __attribute__((aligned(16))) float slse[2][BM];
  __shared__ __attribute__((aligned(16))) float sdel[2][BM];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int N = a.N;
  int kvhead, kblk;
  xcd_map((int)blockIdx.x, a.B * a.Hkv, kvhead, kblk);  // kblk 0 (most rows) first
  const int hk = kvhead % a.Hkv, b = kvhead / a.Hkv;
  const int k0 = kblk * BN;
  const int wk0 = k0 + 32 * wave;     // this wave's first key
  const int key = wk0 + l32;          // the key this lane owns in S/dP

  // the workgroup's K and V rows: B operands of S = Q K^T and dP = dO V^T
  dma_tile<D, BN, kWaves>(head_desc(a.k + a.lk.head(b, hk), N, a.lk.sn, D), k0, a.lk.sn, wave, lane, Ks);
  dma_tile<D, BN, kWaves>(head_desc(a.v + a.lv.head(b, hk), N, a.lv.sn, D), k0, a.lv.sn, wave, lane, Vs);

  f32x16 dk[FB], dv[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[f][i] = 0.0f;
      dv[f][i] = 0.0f;
    }

  // per-lane LDS offsets (elements) that do not change from step to step
  int qa_off[NT];  // Q / dO A operand: row l32, chunk 2t + half
  int ka_off[NT];  // K / V B operand: key row 32*wave + l32, chunk 2t + half
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qa_off[t] = qidx<D>(l32, 16 * t + 8 * half);
    ka_off[t] = qidx<D>(32 * wave + l32, 16 * t + 8 * half);
  }
  const int trow = 4 * (g16 >> 1) + (r16 >> 2);  // transpose reads: row within 16
  int tb_off[FB][2];  // B operand of dV/dK, product t = 0 (rows trow, trow + 8)
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      tb_off[f][e] = qidx<D>(trow + 8 * e, 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3));

  // Steps: every 32-row slice of every query head of the group, from the
  // first row that can see these keys.
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (N - qstart + BM - 1) / BM;
  const int total = nsteps * a.group;
  const int hq0 = hk * a.group;

  StepPos pf{0, qstart};  // the step being copied
  StepPos pc{0, qstart};  // the step being computed
  float stat[3];
  dkdv_load<D>(a, hq0 + pf.h, pf.q0, b, wave, lane, tid, Qs[0], dOs[0], stat);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (tid < BM) bwd_stats_store(stat, pf.q0, tid, N, slse[0], sdel[0]);
  pf.next(qstart, N);
  // d = 128 (one workgroup a CU, registers to spare): the wave's V
  // fragments are read once and kept in registers; d = 64 keeps them in LDS
  // (holding them spills at three workgroups a CU)
  bf16x8 vfr[NT];
  if constexpr (D == 128) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) vfr[t] = *(const bf16x8*)(&Vs[ka_off[t]]);
  }

  for (int s = 0; s < total; ++s) {
    const int cur = s & 1;
    const int q0 = pc.q0;
    // stage s is complete; every wave is done with stage s-1 (copied next)
    __syncthreads();
    const bool more = s + 1 < total;
    const int q0_next = pf.q0;
    dkdv_step<D, CAUSAL>(a, dk, dv, qa_off, ka_off, tb_off, Qs[cur], dOs[cur], Ks, Vs, vfr, slse[cur],
                         sdel[cur], Qs[cur ^ 1], dOs[cur ^ 1], more, hq0 + pf.h, pf.q0, b, wave,
                         lane, tid, stat, q0, wk0, key, half);
    pf.next(qstart, N);
    if (more) {
      // the copies must land before the next barrier publishes the stage
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      if (tid < BM) bwd_stats_store(stat, q0_next, tid, N, slse[cur ^ 1], sdel[cur ^ 1]);
    }
    pc.next(qstart, N);
  }

  // ---- dK = alpha * sum dS^T Q, dV = sum P^T dO for this wave's 32 keys
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = wk0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (kr < N) {
        const int col = 32 * f + l32;
        a.dk[a.ldk.head(b, hk) + (size_t)kr * a.ldk.sn + col] = bf16_bits(a.alpha * dk[f][i]);
        a.dv[a.ldv.head(b, hk) + (size_t)kr * a.ldv.sn + col] = bf16_bits(dv[f][i]);
      }
    }
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  const dim3 grid((unsigned)(((a.N + kDkdvKeys - 1) / kDkdvKeys) * a.Hkv * a.B));
  if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
