// Internal helpers shared by the gfx950 kernels of libusp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace usp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 MFMA: acc[32x32] += A[32x16] * B[16x32].
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32];
// accumulator register i of lane l holds row 8*(i/4) + 4*(l/32) + i%4,
// column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Reduction-axis reordering inside every 16-element chunk. The 8 values a
// lane holds for one 16-wide k-chunk of a 32x32 accumulator (registers 8c..8c+7
// of half h) are the chunk positions {4h..4h+3, 8+4h..8+4h+3}; a key-major copy
// of the other operand stores position p at slot kperm(p) so that a lane reads
// its 8 matching values with one 16-byte load. kperm swaps bits 2 and 3 and is
// its own inverse.
__host__ __device__ __forceinline__ int kperm(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, RNE
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}

// Both halves of a wave64 for one value: after v_permlane32_swap of x with
// itself, lo holds x from lanes 0-31 and hi holds x from lanes 32-63 in every
// lane. The empty asm keeps the two results distinct: given the same value for
// both operands, this compiler otherwise folds hi into lo.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  unsigned a = r[0], b = r[1];
  asm volatile("" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
// Combine a value across the two 32-lane halves of a wave64.
__device__ __forceinline__ float half_swap_max(float x) {
  float lo, hi;
  half_pair(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  float lo, hi;
  half_pair(x, lo, hi);
  return lo + hi;
}

// Document bounds of position i from packed-sequence offsets cu[0..n_docs]
// (binary search; every index stays in [0, n_docs]). Without cu the whole
// padded sequence is one document.
struct DocBounds {
  int lo, hi;  // [lo, hi)
};
__device__ __forceinline__ DocBounds doc_bounds(const int32_t* cu, int n_docs, int i, int s_pad) {
  if (cu == nullptr) return {0, s_pad};
  int a = 0, b = n_docs - 1;  // find largest k in [0, n_docs-1] with cu[k] <= i
  while (a < b) {
    int m = (a + b + 1) >> 1;
    if (cu[m] <= i) a = m; else b = m - 1;
  }
  int lo = cu[a], hi = cu[a + 1];
  lo = lo < 0 ? 0 : (lo > s_pad ? s_pad : lo);
  hi = hi < lo ? lo : (hi > s_pad ? s_pad : hi);
  return {lo, hi};
}

// Key-major workspace row length: padded so every 64-key tile is in bounds.
__host__ __device__ __forceinline__ int64_t kmajor_len(int64_t s_pad) {
  return (s_pad + 127) / 128 * 128;
}

}  // namespace usp
