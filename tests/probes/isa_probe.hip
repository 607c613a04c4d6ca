// isa_probe.hip -- test infrastructure: runs single gfx950 instructions on
// caller-chosen operands so that the tests can check the oracle's models of
// them (bf16, FP8 and FP4 matrix instruction accumulation, exponential).  Not part of the
// library; shares no code with it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One v_mfma_f32_32x32x16_bf16 per wave: a [n][32][16] (row-major A), b
// [n][16][32] (row-major B), c/d [n][32][32] fp32.  Lane l supplies A row
// l%32 and B column l%32 at k = 8*(l/32) .. +7; it holds D column l%32, rows
// 8*(i/4) + 4*(l/32) + i%4 for register i.
__global__ void mfma_bf16_probe(const uint16_t* a, const uint16_t* b, const float* c, float* d) {
  const int w = blockIdx.x, l = threadIdx.x, col = l & 31, kh = l >> 5;
  const uint16_t* A = a + (size_t)w * 512;
  const uint16_t* B = b + (size_t)w * 512;
  const float* C = c + (size_t)w * 1024;
  float* D = d + (size_t)w * 1024;
  bf16x8 av, bv;
  for (int j = 0; j < 8; ++j) {
    av[j] = __builtin_bit_cast(__bf16, A[col * 16 + 8 * kh + j]);
    bv[j] = __builtin_bit_cast(__bf16, B[(8 * kh + j) * 32 + col]);
  }
  f32x16 acc;
  for (int i = 0; i < 16; ++i) acc[i] = C[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  for (int i = 0; i < 16; ++i) D[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col] = acc[i];
}

// One v_mfma_scale_f32_32x32x64_f8f6f4 per wave with E4M3 operands and unit
// scales: a [n][32][64] and b [n][64][32] E4M3 bytes (row-major), c/d
// [n][32][32] fp32.  Lane l supplies A row l%32 and B column l%32 at k =
// 32*(l/32) .. +31 (byte j of its eight words is k = 32*(l/32) + j); the
// result layout is that of the bf16 instruction above.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__global__ void mfma_fp8_probe(const uint8_t* a, const uint8_t* b, const float* c, float* d) {
  const int w = blockIdx.x, l = threadIdx.x, col = l & 31, kh = l >> 5;
  const uint8_t* A = a + (size_t)w * 2048;
  const uint8_t* B = b + (size_t)w * 2048;
  const float* C = c + (size_t)w * 1024;
  float* D = d + (size_t)w * 1024;
  i32x8 av, bv;
  for (int q = 0; q < 8; ++q) {
    uint32_t wa = 0, wb = 0;
    for (int j = 0; j < 4; ++j) {
      const int k = 32 * kh + 4 * q + j;
      wa |= (uint32_t)A[col * 64 + k] << (8 * j);
      wb |= (uint32_t)B[k * 32 + col] << (8 * j);
    }
    av[q] = (int)wa;
    bv[q] = (int)wb;
  }
  f32x16 acc;
  for (int i = 0; i < 16; ++i) acc[i] = C[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col];
  // formats 0, 0: E4M3 operands; scale bytes 127 = 2^0
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  for (int i = 0; i < 16; ++i) D[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col] = acc[i];
}

// One v_mfma_scale_f32_32x32x64_f8f6f4 per wave with E2M1 (FP4) operands:
// a [n][32][64] and b [n][64][32] E2M1 codes (one per byte, low nibble),
// sa [n][32][2] and sb [n][2][32] E8M0 scale bytes (block h = k / 32 of a
// row of A or a column of B), c/d [n][32][32] fp32.  Lane l supplies row /
// column l%32 at k = 32*(l/32) + j in nibble j of its first four words, and
// the scale of that block.
__global__ void mfma_fp4_probe(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                               const float* c, float* d) {
  const int w = blockIdx.x, l = threadIdx.x, col = l & 31, kh = l >> 5;
  const uint8_t* A = a + (size_t)w * 2048;
  const uint8_t* B = b + (size_t)w * 2048;
  const float* C = c + (size_t)w * 1024;
  float* D = d + (size_t)w * 1024;
  i32x8 av = {0, 0, 0, 0, 0, 0, 0, 0}, bv = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int q = 0; q < 4; ++q) {
    uint32_t wa = 0, wb = 0;
    for (int j = 0; j < 8; ++j) {
      const int k = 32 * kh + 8 * q + j;
      wa |= (uint32_t)(A[col * 64 + k] & 15u) << (4 * j);
      wb |= (uint32_t)(B[k * 32 + col] & 15u) << (4 * j);
    }
    av[q] = (int)wa;
    bv[q] = (int)wb;
  }
  const int scale_a = sa[(size_t)w * 64 + col * 2 + kh];
  const int scale_b = sb[(size_t)w * 64 + kh * 32 + col];
  f32x16 acc;
  for (int i = 0; i < 16; ++i) acc[i] = C[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col];
  // formats 4, 4: E2M1 operands; scale bytes in bits 0..7
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, scale_a, 0, scale_b);
  for (int i = 0; i < 16; ++i) D[(8 * (i / 4) + 4 * kh + i % 4) * 32 + col] = acc[i];
}

__global__ void exp2_probe(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}

extern "C" int probe_mfma_bf16(const void* a, const void* b, const void* c, void* d, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_bf16_probe, dim3(n), dim3(64), 0, 0, (const uint16_t*)a, (const uint16_t*)b,
                     (const float*)c, (float*)d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int probe_mfma_fp8(const void* a, const void* b, const void* c, void* d, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_fp8_probe, dim3(n), dim3(64), 0, 0, (const uint8_t*)a, (const uint8_t*)b,
                     (const float*)c, (float*)d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int probe_mfma_fp4(const void* a, const void* b, const void* sa, const void* sb, const void* c,
                              void* d, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_fp4_probe, dim3(n), dim3(64), 0, 0, (const uint8_t*)a, (const uint8_t*)b,
                     (const uint8_t*)sa, (const uint8_t*)sb, (const float*)c, (float*)d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int probe_exp2(const void* x, void* y, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(exp2_probe, dim3((n + 255) / 256), dim3(256), 0, 0, (const float*)x, (float*)y, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
