// attn_internal.h -- device types and launcher declarations shared by the
// HIP translation units of the library (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;

enum Guard { kGuardNone = 0, kGuardBeta = 1, kGuardEps = 2 };

// Tile shape of the streaming forward: 4 waves x 32 query rows per
// workgroup, 64 keys per streaming step (tie decision and shift).  In bf16
// mode Ō is rounded to bf16 after every kFwdRoundN keys and after a row's
// last step.
constexpr int kFwdBlockM = 128;
constexpr int kFwdBlockN = 64;
constexpr int kFwdRoundN = 512;
// Block size of the FA2-as-tensor-operations schedule (attn_fwd_block.hip).
constexpr int kFwdOpsBlockN = 512;
// Products per matrix instruction along every contraction.
constexpr int kMfmaK = 16;

// Element strides of one tensor: batch and head (64-bit), row (32-bit: one
// head's rows are addressed with 32-bit byte offsets); head_dim stride 1.
struct Layout {
  int64_t sb, sh;
  int sn;
  __device__ __forceinline__ size_t head(int b, int h) const {
    return (size_t)((int64_t)b * sb + (int64_t)h * sh);
  }
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* row_m;
  float* row_l;
  uint8_t* row_flags;
  void* obar;      // nullable
  float* row_max;  // nullable
  int B, Hq, Hkv, N, group;
  float alpha;     // softmax scale (fp32)
  float c1;        // fl32(alpha * log2(e))
  float beta, tie_eps, shift_eps;
  int pv_fixed_scale;  // FP8 product: 1 = operand scale fixed at 2^8
  int pv_mx_ceil;      // MXFP4 product: 1 = block scale from ceil(log2 amax)
  Layout lq, lk, lv, lo;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* row_m;
  const float* row_l;
  float* delta;
  float* row_dsum;  // nullable: row sums of dS (dQ kernel)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, Hq, Hkv, N, group;
  float alpha, c1;
  Layout lq, lk, lv, lo, ldo, ldq, ldk, ldv;
};

// Workgroup order on the 8 XCDs (each with its own L2): the hardware hands
// consecutive workgroup ids to XCDs round-robin.  When the number of heads is
// a multiple of 8, head h's blocks all land on XCD h/(heads/8), so one head's
// K/V (forward) or Q/dO (backward) is re-read from one L2.  Within an XCD the
// ids go block-major (block 0 of every head, then block 1, ...), and callers
// number blocks heaviest first, so the longest workgroups of a causal launch
// start first and the tail is short.
// Returns (head index, block index) for linear workgroup id L.
__device__ __forceinline__ void xcd_map(int L, int heads, int& head, int& blk) {
  constexpr int kXcds = 8;
  if (heads % kXcds == 0) {
    const int hpx = heads / kXcds;
    const int xcd = L % kXcds, local = L / kXcds;
    blk = local / hpx;
    head = xcd * hpx + local % hpx;
  } else {
    blk = L / heads;
    head = L % heads;
  }
}

// pv: the operands of Ō's product, 0 bf16, 1 FP8 E4M3, 2 MXFP4
hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int guard, bool obar_f32,
                      int pv, hipStream_t s);
hipError_t launch_fwd_block(const FwdArgs& a, int d, bool causal, int guard, bool obar_f32,
                            bool untiled, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool causal, bool delta_dp, hipStream_t s);

// Query rows per inner step of the dK/dV kernel.
constexpr int kBwdBlockM = 32;

}  // namespace attn
