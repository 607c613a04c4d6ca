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

// Roles of the four waves of a workgroup.  Every wave computes S, dP, P, dS,
// dV and dK for its own 32 keys.  Beyond that, waves 0-1 ("loaders") fetch
// the next steps' Q and dO rows and statistics into the LDS stages, and
// waves 2-3 ("dQ waves") compute the previous step's dQ rows and add them
// with global atomics.  A wait for a fetch also waits for every atomic its
// wave issued before (one counter covers both), and atomics queue at the L2;
// with the roles split no wave ever waits for an atomic inside the loop.
constexpr int kBwdLoaders = 2;
// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt vmcnt(0) with the other counters left free.
constexpr int kWaitVmcnt0 = 0x0F70;

// One step = 32 query rows of one query head of the group.  The loaders copy
// its Q and dO rows straight into one of the two LDS stages with buffer
// loads to LDS (16 bytes a lane, a wave's 64 lanes filling 1 KiB of the tile
// in lane order; each lane picks the global chunk that belongs at its tile
// position under the swizzle).  Rows past the sequence end lie outside the
// buffer's range and read as zeros.
template <int D>
__device__ __forceinline__ void bwd_load(const BwdArgs& a, int hq, int q0, int b, int lw,
                                         int lane, uint16_t* Qs, uint16_t* dOs) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int CPR = D / 8;                                  // 16-byte chunks per row
  constexpr int NI = kBwdBlockM * CPR / 64 / kBwdLoaders;     // 1 KiB pieces per loader per tensor
  const size_t hoff = ((size_t)(b * a.Hq + hq) * a.N) * D;
  const int nbytes = a.N * D * 2;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + hoff), 0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rg =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + hoff), 0, nbytes, kBufferWord3);
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int piece = lw * NI + u;
    const int p = piece * 64 + lane;                // chunk position in the tile
    const int row = p / CPR;
    const int c = (p % CPR) ^ qswz(row);            // logical chunk stored there
    const int voff = ((q0 + row) * D + 8 * c) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(Qs + piece * 512), 16, voff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void*)(dOs + piece * 512), 16, voff, 0, 0, 0);
  }
}

// Row statistics of a step (threads 0..31 of wave 0): raw loads, then the
// log2-domain shift once they have arrived.
struct BwdStats {
  float m, l, del;
};

__device__ __forceinline__ void bwd_stats_load(const BwdArgs& a, int hq, int q0, int b, int tid,
                                               BwdStats& st) {
  const size_t r = (size_t)(b * a.Hq + hq) * a.N + q0 + tid;
  st.m = 0.0f;
  st.l = 1.0f;
  st.del = 0.0f;
  if (q0 + tid < a.N) {
    st.m = a.row_m[r];
    st.l = a.row_l[r];
    st.del = a.delta[r];
  }
}

__device__ __forceinline__ void bwd_stats_store(int tid, const BwdStats& st, float* slse,
                                                float* sdel) {
  // P = exp(t - m) / l = exp2(t*log2(e) - lse2); a row whose every weight
  // underflowed (l == 0) keeps P = NaN, as 0 * (1/0) gives
  slse[tid] = st.l > 0.0f ? __builtin_fmaf(st.m, kLog2e, __builtin_log2f(st.l))
                          : __builtin_nanf("");
  sdel[tid] = st.del;
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

// dQ[q0..q0+31][D/2 features from f0] += dS K over the workgroup's 128 keys
// (v_mfma_f32_16x16x32_bf16 on 16x16 tiles; key blocks with no visible key
// hold zeros in the dS tile), one atomic add per element.  K comes from the
// workgroup's K tile through the transpose read.  dQ has whole 32-row steps
// per head (rows past the sequence end receive zeros and are never read).
template <int D>
__device__ __forceinline__ void bwd_dq(const uint16_t* ds, const uint16_t* ks, float* dQ, int q0,
                                       int f0, int g16, int r16) {
  constexpr int NJ = D / 32;  // 16-feature tiles
  f32x4 acc[2][NJ];
#pragma unroll
  for (int mq = 0; mq < 2; ++mq)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mq][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one 32-key block at a time: its dS rows (A) and K columns (B)
#pragma unroll
  for (int kb = 0; kb < kBwdKB; ++kb) {
    const int kk = 32 * kb + 8 * g16 + (r16 >> 2);
    bf16x8 da[2], kq[NJ];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      // A = dS[rows 16mq + r16][keys 32kb + 8*g16 + 0..7]
      const int u = 4 * mq + (r16 & 3);
      da[mq] = frag2(lds_read_tr(ds + didx(kk, u)), lds_read_tr(ds + didx(kk + 4, u)));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // B = K[keys 32kb + 8*g16 + 0..7][f0 + 16j + r16]
      const int col = f0 + 16 * j + 4 * (r16 & 3);
      kq[j] = frag2(lds_read_tr(ks + qidx<D>(kk, col)), lds_read_tr(ks + qidx<D>(kk + 4, col)));
    }
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[mq][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[mq], kq[j], acc[mq][j], 0, 0, 0);
  }
#pragma unroll
  for (int mq = 0; mq < 2; ++mq)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // C register i holds row q0 + 16mq + 4*g16 + i
      float* dst = dQ + (size_t)(q0 + 16 * mq + 4 * g16) * D + f0 + 16 * j + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + (size_t)i * D, acc[mq][j][i]);
    }
}

// Everything one wave does for one step after the stage barrier: S, dP, P,
// dS (written key-major to the step's dS tile), dV and dK for its keys, and
// for a dQ wave the previous step's dQ, in one block so that the two
// interleave.
template <int D, bool CAUSAL, bool DQW>
__device__ __forceinline__ void bwd_step(
    const BwdArgs& a, f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
    const int (&qa_off)[D / kMfmaK], const int (&ka_off)[D / kMfmaK], const int (&tb_off)[D / 32],
    const uint16_t* qs, const uint16_t* gs, const float* slse, const float* sdel, uint16_t* dsw,
    const uint16_t* dsp, const uint16_t* ks, const uint16_t* vs, float* dqp, int qp, int f0, int q0,
    int wk0, int key, int kl, int half, int l32, int g16, int r16) {
  constexpr int BM = kBwdBlockM;
  constexpr int NT = D / kMfmaK;
  constexpr int FB = D / 32;
  const int N = a.N;
  const bool live = wk0 < N && (!CAUSAL || q0 + BM - 1 >= wk0);
  if (!live) {
    // no key of this wave is visible to these rows: its dS columns are zero
#pragma unroll
    for (int u = 0; u < 4; ++u) *(uint2*)(&dsw[didx(kl, 2 * u + half)]) = make_uint2(0, 0);
    if (DQW) bwd_dq<D>(dsp, ks, dqp, qp, f0, g16, r16);
    return;
  }
  // ---- S = Q K^T and dP = dO V^T: lane = key, register i = row 8(i/4)+4*half+i%4
  f32x16 sv, dp;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sv[i] = 0.0f;
    dp[i] = 0.0f;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // B operands: this lane's key row of K and V, features 16t + 8*half + 0..7
    const bf16x8 kb = *(const bf16x8*)(&ks[ka_off[t]]);
    const bf16x8 vb = *(const bf16x8*)(&vs[ka_off[t]]);
    const bf16x8 qa = *(const bf16x8*)(&qs[qa_off[t]]);
    sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, sv, 0, 0, 0);
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
  // (row q0 + 4*half + r_i, r_i = 8(i/4) + i%4) is visible iff lo <= r_i < hi
  const bool edge = (CAUSAL && wk0 + 31 > q0) || q0 + BM > N || wk0 + 32 > N;
  if (__builtin_expect(edge, 0)) {
    // an empty volatile asm keeps this block a branch: the compiler would
    // otherwise turn it into selects executed on every step
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
  // ---- dV += P^T dO and dK += dS^T Q, contraction over the 32 rows: the k
  // index 8*half + j of product t is row 16t + 8(j/4) + 4*half + j%4, so the
  // B operand is two transpose reads of 4 rows each
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
  if (DQW) {
    // keep the dQ work after this step's (the scheduler would otherwise
    // hoist its reads into the softmax and exceed the register budget)
    __builtin_amdgcn_sched_barrier(0);
    bwd_dq<D>(dsp, ks, dqp, qp, f0, g16, r16);
  }
}

// d = 64: two workgroups per CU (two waves per SIMD, at most 256 VGPRs a
// wave); d = 128 needs more registers and runs one.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_main_kernel(BwdArgs a) {
  constexpr int BN = kBwdKeys;
  constexpr int BM = kBwdBlockM;     // query rows per step (32)
  constexpr int NT = D / kMfmaK;     // 16-wide steps along d
  constexpr int FB = D / 32;         // 32-feature blocks of dK/dV

  // two stages: step s computes from stage s&1 while step s+1 is written
  // to the other; the dS tile is double-buffered the same way
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[2][BN * BM];
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
  const size_t kvoff = ((size_t)(b * a.Hkv + hk) * N) * D;
  const uint16_t* __restrict__ K = a.k + kvoff;
  const uint16_t* __restrict__ V = a.v + kvoff;

  // the workgroup's K and V rows, row-major (swizzled like the stages): the
  // B operands of S = Q K^T and dP = dO V^T, and K for the dQ product
#pragma unroll
  for (int u = 0; u < BN * D / 8 / kThreads; ++u) {
    const int c = tid + u * kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (k0 + row < N) {
      kr = *(const uint4*)(K + (size_t)(k0 + row) * D + col);
      vr = *(const uint4*)(V + (size_t)(k0 + row) * D + col);
    }
    *(uint4*)(&Ks[qidx<D>(row, col)]) = kr;
    *(uint4*)(&Vs[qidx<D>(row, col)]) = vr;
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
  int ka_off[NT];  // K/V B operand: key row 32*wave + l32, chunk 2t + half
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qa_off[t] = qidx<D>(l32, 16 * t + 8 * half);
    ka_off[t] = qidx<D>(32 * wave + l32, 16 * t + 8 * half);
  }
  const int trow = 4 * (g16 >> 1) + (r16 >> 2);  // transpose reads: row within 16
  int tb_off[FB];  // B operand of dV/dK, product t = 0; t = 1 is 16 rows on
#pragma unroll
  for (int f = 0; f < FB; ++f) tb_off[f] = qidx<D>(trow, 32 * f + 16 * (g16 & 1) + 4 * (r16 & 3));
  const int kl = 32 * wave + l32;  // this lane's key within the tile
  const bool loader = wave < kBwdLoaders;
  const int f0 = (D / 2) * (wave - kBwdLoaders);  // dQ waves: first of their D/2 features

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
  // the dQ of step 0 reads "step -1"'s tile: zeros, added to step 0's rows
#pragma unroll
  for (int u = 0; u < BN * BM / 8 / kThreads; ++u)
    *(uint4*)(&dSt[1][8 * (tid + u * kThreads)]) = make_uint4(0, 0, 0, 0);
  BwdStats st;
  if (loader) {
    bwd_load<D>(a, hq0 + pf.h, pf.q0, b, wave, lane, Qs[0], dOs[0]);
    if (tid < BM) {
      bwd_stats_load(a, hq0 + pf.h, pf.q0, b, tid, st);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      bwd_stats_store(tid, st, slse[0], sdel[0]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  pf.next(qstart, N);

  for (int s = 0; s < total; ++s) {
    const int cur = s & 1;
    // stage s and step s-1's dS tile are complete; every wave is done with
    // step s-1's stage (written next) and with the dS tile that step s-2's
    // dQ read (written below)
    __syncthreads();
    // loaders: step s+1 goes to the other stage while step s computes
    const bool more = s + 1 < total;
    if (loader && more) {
      bwd_load<D>(a, hq0 + pf.h, pf.q0, b, wave, lane, Qs[cur ^ 1], dOs[cur ^ 1]);
      if (tid < BM) bwd_stats_load(a, hq0 + pf.h, pf.q0, b, tid, st);
    }
    pf.next(qstart, N);
    float* const dqp = dq_base + (size_t)(hq0 + pp.h) * a.Npad * D;
    if (loader)
      bwd_step<D, CAUSAL, false>(a, dk, dv, qa_off, ka_off, tb_off, Qs[cur], dOs[cur], slse[cur],
                                 sdel[cur], dSt[cur], dSt[cur ^ 1], Ks, Vs, dqp, pp.q0, f0,
                                 pc.q0, wk0, key, kl, half, l32, g16, r16);
    else
      bwd_step<D, CAUSAL, true>(a, dk, dv, qa_off, ka_off, tb_off, Qs[cur], dOs[cur], slse[cur],
                                sdel[cur], dSt[cur], dSt[cur ^ 1], Ks, Vs, dqp, pp.q0, f0, pc.q0,
                                wk0, key, kl, half, l32, g16, r16);
    if (loader && more) {
      // the copies must land before the next barrier publishes the stage
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      if (tid < BM) bwd_stats_store(tid, st, slse[cur ^ 1], sdel[cur ^ 1]);
    }
    if (s > 0) pp.next(qstart, N);
    pc.next(qstart, N);
  }
  __syncthreads();
  if (!loader)
    bwd_dq<D>(dSt[(total - 1) & 1], Ks, dq_base + (size_t)(hq0 + pp.h) * a.Npad * D, pp.q0, f0,
              g16, r16);

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
