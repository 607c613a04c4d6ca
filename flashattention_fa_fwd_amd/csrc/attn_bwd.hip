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
//   * per step of 32 query rows, Q and dO are staged row-major in one of two
//     LDS buffers (one barrier per step: step s computes from one buffer
//     while step s+1 is written to the other);
//   * S = Q K^T and dP = dO V^T come out with lane = key and registers =
//     query rows, the A-operand layout of dV += P^T dO and dK += dS^T Q; the
//     B operands (dO and Q with the contraction over rows) come from the
//     row-major tiles through the gfx950 LDS transpose read;
//   * dS is written key-major (four rows per 8-byte write) into a
//     double-buffered tile; the next step, each wave reads it back through
//     the transpose read as the A operand of a 16-feature slice of dQ over
//     the 128 keys (v_mfma_f32_16x16x32_bf16, K slice held in registers) and
//     adds it to the fp32 accumulator with one atomic per element;
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
    float* dq = a.dq_acc + ((row / a.N) * a.Npad + row % a.N) * D + part * EPT;
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
  const size_t row = 4 * i / D;
  const f32x4 v = *(const f32x4*)(a.dq_acc + ((row / a.N) * a.Npad + row % a.N) * D + 4 * i % D);
  const uint32_t lo = bf16_bits(a.alpha * v[0]) | ((uint32_t)bf16_bits(a.alpha * v[1]) << 16);
  const uint32_t hi = bf16_bits(a.alpha * v[2]) | ((uint32_t)bf16_bits(a.alpha * v[3]) << 16);
  *(uint2*)(a.dq + 4 * i) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- bwd_main
// LDS transpose read (gfx950): within each group of 16 lanes, lane r supplies
// the address of 4 consecutive bf16 E_r; lane i receives E_{4j + i/4}[i%4]
// for j = 0..3.  If lane r points at row k0 + r/4, columns n0 + 4(r%4)..+3 of
// a matrix X, lane i receives X[k0 + 0..3][n0 + i]: four consecutive
// contraction indices of one row or column, half of an MFMA operand.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_u16*)p));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ bf16x8 frag2(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Q / dO stage tiles: row r of D bf16, its 16-byte chunk c stored at chunk
// c ^ qswz(r).  Eight consecutive rows reading one chunk (the A-operand
// reads) and four consecutive rows reading two adjacent chunks (the
// transpose reads) then hit 8 distinct 16-byte bank groups.
__device__ __forceinline__ int qswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
template <int D>
__device__ __forceinline__ int qidx(int r, int col) {  // col % 4 == 0
  return r * D + ((((col >> 3) ^ qswz(r))) << 3) + (col & 7);
}

// dS tile, key-major: key k (0..127) holds the 32 rows of the step as eight
// 8-byte units (rows 4u..4u+3), unit u stored at u ^ dswz(k).  Sixteen
// consecutive keys writing one unit, and four consecutive keys read at four
// adjacent units (transpose reads), then use distinct banks.
__device__ __forceinline__ int dswz(int k) { return (((k >> 1) & 1) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int didx(int k, int u) { return k * kBwdBlockM + 4 * (u ^ dswz(k)); }

// One step = 32 query rows of one query head of the group.  Its Q and dO
// rows and the rows' statistics are fetched into registers one step ahead
// and then written to one of two LDS stages.
template <int D>
struct BwdStep {
  static constexpr int CPT = kBwdBlockM * D / 8 / kThreads;  // 16-byte chunks per thread
  uint4 q[CPT], g[CPT];
  float m, l, del;  // threads 0..31: the row's shift, denominator and delta
};

template <int D>
__device__ __forceinline__ void bwd_fetch(const BwdArgs& a, int hq, int q0, int b, int tid,
                                          BwdStep<D>& st) {
  const int N = a.N;
  const size_t qoff = ((size_t)(b * a.Hq + hq) * N) * D;
#pragma unroll
  for (int u = 0; u < BwdStep<D>::CPT; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    st.q[u] = make_uint4(0, 0, 0, 0);
    st.g[u] = make_uint4(0, 0, 0, 0);
    if (q0 + row < N) {
      st.q[u] = *(const uint4*)(a.q + qoff + (size_t)(q0 + row) * D + col);
      st.g[u] = *(const uint4*)(a.dout + qoff + (size_t)(q0 + row) * D + col);
    }
  }
  // raw loads only: nothing here waits for them (a wait would also wait for
  // every atomic issued before)
  if (tid < kBwdBlockM) {
    const size_t r = (size_t)(b * a.Hq + hq) * N + q0 + tid;
    st.m = 0.0f;
    st.l = 1.0f;
    st.del = 0.0f;
    if (q0 + tid < N) {
      st.m = a.row_m[r];
      st.l = a.row_l[r];
      st.del = a.delta[r];
    }
  }
}

template <int D>
__device__ __forceinline__ void bwd_stage(int tid, const BwdStep<D>& st, uint16_t* Qs,
                                          uint16_t* dOs, float* slse, float* sdel) {
#pragma unroll
  for (int u = 0; u < BwdStep<D>::CPT; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(uint4*)(&Qs[qidx<D>(row, col)]) = st.q[u];
    *(uint4*)(&dOs[qidx<D>(row, col)]) = st.g[u];
  }
  if (tid < kBwdBlockM) {
    // P = exp(t - m) / l = exp2(t*log2(e) - lse2); a row whose every weight
    // underflowed (l == 0) keeps P = NaN, as 0 * (1/0) gives
    slse[tid] = st.l > 0.0f ? __builtin_fmaf(st.m, kLog2e, __builtin_log2f(st.l))
                            : __builtin_nanf("");
    sdel[tid] = st.del;
  }
}

constexpr int kBwdKeys = 128;          // keys per workgroup (32 per wave)
constexpr int kBwdKB = kBwdKeys / 32;  // 32-key blocks per workgroup

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

// dQ[q0..q0+31][this wave's features] += dS K over the workgroup's 128 keys
// (v_mfma_f32_16x16x32_bf16; key blocks with no visible key hold zeros),
// one atomic add per element.  dQ has whole 32-row steps per head (rows past
// the sequence end receive zeros and are never read).
template <int D, int DQB>
__device__ __forceinline__ void bwd_dq(const uint16_t* ds,
                                       const bf16x8 (&kq)[DQB][kBwdKB], float* dQ, int q0,
                                       int wave, int g16, int r16) {
#pragma unroll
  for (int sl = 0; sl < DQB; ++sl) {
    const int d0 = 16 * (wave * DQB + sl);
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      // A = dS[rows 16mq + r16][keys 32kb + 8*g16 + 0..7]
      bf16x8 da[kBwdKB];
#pragma unroll
      for (int kb = 0; kb < kBwdKB; ++kb) {
        const int kk = 32 * kb + 8 * g16 + (r16 >> 2);
        const int u = 4 * mq + (r16 & 3);
        da[kb] = frag2(lds_read_tr(ds + didx(kk, u)), lds_read_tr(ds + didx(kk + 4, u)));
      }
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kBwdKB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[kb], kq[sl][kb], acc, 0, 0, 0);
      // C register i holds row q0 + 16mq + 4*g16 + i
      float* dst = dQ + (size_t)(q0 + 16 * mq + 4 * g16) * D + d0 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + (size_t)i * D, acc[i]);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdArgs a) {
  constexpr int BN = kBwdKeys;
  constexpr int BM = kBwdBlockM;     // query rows per step (32)
  constexpr int NT = D / kMfmaK;     // 16-wide steps along d
  constexpr int FB = D / 32;         // 32-feature blocks of dK/dV
  constexpr int DQB = D / 16 / 4;    // 16-feature dQ slices per wave (1 or 2)
  constexpr int KB = kBwdKB;

  // two stages: step s computes from stage s&1 while step s+1 is written
  // to the other; the dS tile is double-buffered the same way
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[2][BN * BM];
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
  const size_t kvoff = ((size_t)(b * a.Hkv + hk) * N) * D;
  const uint16_t* __restrict__ K = a.k + kvoff;
  const uint16_t* __restrict__ V = a.v + kvoff;

  // K and V rows of this lane's key as B operands of S = Q K^T and
  // dP = dO V^T: [16t + 8*half + 0..7]
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
  // K as the B operand of this wave's dQ slices: lane holds
  // K[k0 + 32kb + 8*g16 + 0..7][d0 + r16] for every 32-key block kb
  bf16x8 kq[DQB][KB];
#pragma unroll
  for (int sl = 0; sl < DQB; ++sl)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int d0 = 16 * (wave * DQB + sl);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = k0 + 32 * kb + 8 * g16 + 2 * j;
        const uint32_t lo = kk < N ? K[(size_t)kk * D + d0 + r16] : 0u;
        const uint32_t hi = kk + 1 < N ? K[(size_t)(kk + 1) * D + d0 + r16] : 0u;
        w[j] = lo | (hi << 16);
      }
      kq[sl][kb] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }

  f32x16 dk[FB], dv[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[f][i] = 0.0f;
      dv[f][i] = 0.0f;
    }

  // per-lane LDS offsets (elements) that do not change from step to step
  int qa_off[NT];  // A operand: row l32, chunk 2t + half
#pragma unroll
  for (int t = 0; t < NT; ++t) qa_off[t] = qidx<D>(l32, 16 * t + 8 * half);
  const int trow = 4 * (g16 >> 1) + (r16 >> 2);  // transpose reads: row within 16
  int tb_off[FB];  // B operand of dV/dK, product t = 0; t = 1 is 16 rows on
#pragma unroll
  for (int f = 0; f < FB; ++f) tb_off[f] = qidx<D>(trow, 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3));
  const int kl = 32 * wave + l32;  // this lane's key within the tile

  // Steps: every 32-row slice of every query head of the group, from the
  // first row that can see these keys.
  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (N - qstart + BM - 1) / BM;
  const int total = nsteps * a.group;
  const int hq0 = hk * a.group;
  float* const dq_base = a.dq_acc + (size_t)b * a.Hq * a.Npad * D;

  StepPos pf{0, qstart};  // the step being fetched
  StepPos pc{0, qstart};  // the step being computed
  StepPos pp{0, qstart};  // the step whose dQ is being added
  // the dQ block of step 0 reads "step -1"'s tile: zeros, added to step 0's rows
#pragma unroll
  for (int u = 0; u < BN * BM / 8 / kThreads; ++u)
    *(uint4*)(&dSt[1][8 * (tid + u * kThreads)]) = make_uint4(0, 0, 0, 0);
  BwdStep<D> st;
  bwd_fetch<D>(a, hq0 + pf.h, pf.q0, b, tid, st);
  bwd_stage<D>(tid, st, Qs[0], dOs[0], slse[0], sdel[0]);
  pf.next(qstart, N);
  if (total > 1) bwd_fetch<D>(a, hq0 + pf.h, pf.q0, b, tid, st);
  pf.next(qstart, N);

  for (int s = 0; s < total; ++s) {
    const int cur = s & 1;
    const int q0 = pc.q0;
    // stage s and step s-1's dS tile are complete; every wave is done with
    // step s-1's stage (written next) and with the dS tile that step s-2's
    // dQ read (written below)
    __syncthreads();
    // Waiting for a fetch also waits for every global atomic issued before
    // the wait (the counter covers both), so the order is: stage the step
    // fetched one iteration ago, issue the next fetch and the previous
    // step's dQ atomics together, and compute while both are in flight.
    if (s + 1 < total) {
      bwd_stage<D>(tid, st, Qs[cur ^ 1], dOs[cur ^ 1], slse[cur ^ 1], sdel[cur ^ 1]);
      if (s + 2 < total) bwd_fetch<D>(a, hq0 + pf.h, pf.q0, b, tid, st);
      pf.next(qstart, N);
    }
    // dQ of the previous step: issued inside both branches below, so its
    // matrix and memory work interleaves with this step's
    const uint16_t* dsp = dSt[cur ^ 1];
    float* const dqp = dq_base + (size_t)(hq0 + pp.h) * a.Npad * D;

    uint16_t* dsw = dSt[cur];
    const bool live = wk0 < N && (!CAUSAL || q0 + BM - 1 >= wk0);
    if (live) {
      const uint16_t* qs = Qs[cur];
      const uint16_t* gs = dOs[cur];
      // ---- S = Q K^T and dP = dO V^T: lane = key, register i = row 8(i/4)+4*half+i%4
      f32x16 sv, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = 0.0f;
        dp[i] = 0.0f;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 qa = *(const bf16x8*)(&qs[qa_off[t]]);
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[t], sv, 0, 0, 0);
        const bf16x8 ga = *(const bf16x8*)(&gs[qa_off[t]]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[t], dp, 0, 0, 0);
      }
      bwd_dq<D, DQB>(dsp, kq, dqp, pp.q0, wave, g16, r16);
      // ---- P = exp2(s * alpha*log2(e) - lse2) and dS = P (dP - delta)
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rl = 8 * g + 4 * half;  // first of the 4 rows of this group
        const f32x4 lv = *(const f32x4*)(&slse[cur][rl]);
        const f32x4 dl = *(const f32x4*)(&sdel[cur][rl]);
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
        const uint32_t p0 = pack_bf16(pv[8 * t + 0], pv[8 * t + 1]);
        const uint32_t p1 = pack_bf16(pv[8 * t + 2], pv[8 * t + 3]);
        const uint32_t p2 = pack_bf16(pv[8 * t + 4], pv[8 * t + 5]);
        const uint32_t p3 = pack_bf16(pv[8 * t + 6], pv[8 * t + 7]);
        pa[t] = __builtin_bit_cast(bf16x8, make_uint4(p0, p1, p2, p3));
        const uint32_t s0 = pack_bf16(dsv[8 * t + 0], dsv[8 * t + 1]);
        const uint32_t s1 = pack_bf16(dsv[8 * t + 2], dsv[8 * t + 3]);
        const uint32_t s2 = pack_bf16(dsv[8 * t + 4], dsv[8 * t + 5]);
        const uint32_t s3 = pack_bf16(dsv[8 * t + 6], dsv[8 * t + 7]);
        sa[t] = __builtin_bit_cast(bf16x8, make_uint4(s0, s1, s2, s3));
        // dS key-major: rows 16t + 4*half + 0..3 (unit 4t + half) and 8 on
        *(uint2*)(&dsw[didx(kl, 4 * t + half)]) = make_uint2(s0, s1);
        *(uint2*)(&dsw[didx(kl, 4 * t + 2 + half)]) = make_uint2(s2, s3);
      }
      // ---- dV += P^T dO and dK += dS^T Q, contraction over the 32 rows:
      // the k index 8*half + j of product t is row 16t + 8(j/4) + 4*half + j%4,
      // so the B operand is two transpose reads of 4 rows each
#pragma unroll
      for (int f = 0; f < FB; ++f) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int o = tb_off[f] + 16 * t * D;  // rows 16t + trow (row & 7 unchanged)
          const bf16x8 gb = frag2(lds_read_tr(gs + o), lds_read_tr(gs + o + 8 * D));
          dv[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], gb, dv[f], 0, 0, 0);
          const bf16x8 qb = frag2(lds_read_tr(qs + o), lds_read_tr(qs + o + 8 * D));
          dk[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], qb, dk[f], 0, 0, 0);
        }
      }
    } else {
      // no key of this wave is visible to these rows: its dS columns are zero
#pragma unroll
      for (int u = 0; u < 4; ++u) *(uint2*)(&dsw[didx(kl, 2 * u + half)]) = make_uint2(0, 0);
      bwd_dq<D, DQB>(dsp, kq, dqp, pp.q0, wave, g16, r16);
    }
    if (s > 0) pp.next(qstart, N);
    pc.next(qstart, N);
  }
  __syncthreads();
  bwd_dq<D, DQB>(dSt[(total - 1) & 1], kq, dq_base + (size_t)(hq0 + pp.h) * a.Npad * D, pp.q0,
                 wave, g16, r16);

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
