// attn_device.h -- device helpers shared by the HIP kernels of the library:
// bf16 packing, the gfx950 LDS transpose read, the swizzled layout of the
// LDS tiles, and buffer-to-LDS copies of row tiles.  Not part of the ABI.
#pragma once
#include "attn_internal.h"

namespace attn {
namespace {

// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt vmcnt(0) with the other counters left free.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

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

// LDS tiles of D-wide bf16 rows: the 16-byte chunk c of row r is stored at
// chunk c ^ qswz(r).  The gfx950 LDS has 64 four-byte banks; a 16-byte-per-
// lane read is served 16 lanes at a time and a transpose read 32 at a time.
// The permutation (row bits 1..3, and bit 0 for 256-byte rows) makes both
// patterns the kernels use hit 16 distinct 16-byte bank groups: 16
// consecutive rows reading one chunk (row operands) and 4 consecutive rows
// reading 4 adjacent chunks (transpose reads).
template <int D>
__device__ __forceinline__ int qswz(int r) {
  const int s = (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return D == 64 ? s : (s | ((r & 1) << 3));
}
template <int D>
__device__ __forceinline__ int qidx(int r, int col) {  // col % 4 == 0
  return r * D + ((((col >> 3) ^ qswz<D>(r))) << 3) + (col & 7);
}

// Buffer resource (gfx9 layout) of one head's rows: n rows of d bf16, sn
// elements apart, from base; offsets at or past ((n-1)*sn + d)*2 bytes read
// as zeros (row n and later: sn >= d).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 head_desc(const uint16_t* base, int n, int sn, int d) {
  const uint64_t a = (uint64_t)base;
  // uniform by construction; readfirstlane keeps it in scalar registers
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(((n - 1) * sn + d) * 2), kBufferWord3};
}

// One buffer-to-LDS load of 16 bytes a lane: lane i's bytes land at LDS
// address lds_base + 16 i.  Issued as inline assembly so that the compiler
// does not treat it as a write to shared memory in flight: it would wait
// for the copy before every later LDS read, while the copy only ever fills
// the stage that the next step reads.  Callers wait for it (vmcnt) before
// the barrier that publishes the stage.
__device__ __forceinline__ void lds_dma16(i32x4 desc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(desc)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  return (uint32_t)(uintptr_t)(lds_u16*)p;
}

// Copy rows [r0, r0 + ROWS) of a [n, D] bf16 array with row stride sn
// (elements) into a swizzled LDS tile: a wave's 64 lanes fill 1 KiB of the
// tile in lane order (16 bytes a lane), each lane fetching the global chunk
// that belongs at its tile position.  Rows past n lie outside the buffer and
// read as zeros.  Wave w of NW takes its share of the 1 KiB pieces.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(i32x4 desc, int r0, int sn, int w, int lane, uint16_t* tile) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int PIECES = ROWS * CPR / 64;    // 1 KiB pieces per tile
  static_assert(PIECES % NW == 0, "tile / wave split");
#pragma unroll
  for (int u = 0; u < PIECES / NW; ++u) {
    const int piece = w * (PIECES / NW) + u;
    const int p = piece * 64 + lane;          // chunk position in the tile
    const int row = p / CPR;
    const int c = (p % CPR) ^ qswz<D>(row);   // logical chunk stored there
    const int voff = ((r0 + row) * sn + 8 * c) * 2;
    lds_dma16(desc, __builtin_amdgcn_readfirstlane(lds_addr(tile + piece * 512)), voff);
  }
}

}  // namespace
}  // namespace attn
