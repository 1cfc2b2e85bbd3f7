// Internal helpers shared by the gfx950 kernels of libusp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "usp_internal.h"

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

// Slot of 16-byte chunk c in a 256-byte LDS row r (16 chunks): c ^ swz16(r).
// swz16 rotates the low four row bits by two, so both access patterns of the
// attention tiles touch 16 distinct slots: one chunk of 16 consecutive rows
// (row-major fragment reads) and 4 consecutive chunks of 4 consecutive rows
// starting at a multiple of 4 (transposed reads).
__host__ __device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// The same for 128-byte rows (8 chunks; two rows share a 256-byte bank line,
// row r in half r & 1): c ^ swz8(r) with swz8 = (r1, r3, r2) from row bits
// r1..r3. For one row parity it is a bijection of r >> 1, so one chunk of 16
// consecutive rows hits 16 distinct slots; rows 4m + e and 4m + e + 2 differ in
// bit 2, so 4 consecutive chunks (4-aligned) of 4 consecutive rows (4-aligned)
// fill the two halves of both bank lines.
__host__ __device__ __forceinline__ int swz8(int r) {
  return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}
// Chunk swizzle of a tile with D-element bf16 rows (D = 128 or 64).
template <int D>
__host__ __device__ __forceinline__ int swz_row(int r) {
  static_assert(D == 128 || D == 64, "head dim 64 or 128");
  if constexpr (D == 128) return swz16(r);
  else return swz8(r);
}

// Transposed LDS read (ds_read_b64_tr_b16). Lanes act in groups of 16: each
// names 4 consecutive bf16 values, and lane i of a group receives value i%4
// of the values named by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its
// group, in that order.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_v;
__device__ __forceinline__ bf16x4_v lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4_v*)(const_cast<__bf16*>(p)));
}

// Element offset, in a tile of D-element rows stored with swz_row<D>, that
// lane `lane` names in transposed read h (0 or 1) of column block b, for the
// 16-row chunk at row 0. Reads h = 0 and h = 1 together give the lane column
// 32b + lane%32 of rows 8h + 4(lane/32) + j, j = 0..3: the 32x32x16 operand
// (m = column, k = row) in the k-order in which the other operand leaves a
// 32x32 accumulator (see kperm).
template <int D>
__device__ __forceinline__ int tr_offset(int lane, int b, int h) {
  const int r = 8 * h + 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int c = 4 * b + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  return r * D + ((c ^ swz_row<D>(r)) << 3) + 4 * (lane & 1);
}
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* tile, int off0, int off1) {
  const bf16x4_v a = lds_read_tr(tile + off0), b = lds_read_tr(tile + off1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct global->LDS loads issued as inline asm (global_load_lds with a
// scalar 64-bit base, a 32-bit lane offset and the LDS destination in M0).
// The compiler does not see these as memory operations, so it neither waits
// for them at every barrier nor in front of LDS reads it cannot tell apart
// from the destination; the caller waits with vmcnt before the barrier that
// publishes the data. Every direct load of a kernel that uses these must go
// through them (M0 is written here behind the compiler's back).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_lds_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Transposed read (see lds_read_tr) of the pair at byte addresses a0, a1.
__device__ __forceinline__ bf16x8 frag_tr_at(uint32_t a0, uint32_t a1) {
  typedef __attribute__((address_space(3))) bf16x4_v* lp;
  const bf16x4_v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lp)(uintptr_t)a0);
  const bf16x4_v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lp)(uintptr_t)a1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// 16-byte LDS read at byte address a. With a = base + constant, the constant
// goes into the instruction's 16-bit offset field when it fits.
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)a;
}
// LDS byte address of a pointer into a __shared__ array, made wave-uniform
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p));
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
// Maximum of the 32 values of two accumulator tiles as a tree of 3-input
// maxima (16 v_max3_f32, depth 4). The kernels are built without NaN
// semantics (no NaN can arise: masked scores are -inf and every -inf - -inf
// is guarded), so no canonicalising instructions are inserted.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max_of_32(const f32x16& x, const f32x16& y) {
  float l1[12];
#pragma unroll
  for (int g = 0; g < 5; ++g) l1[g] = max3f(x[3 * g], x[3 * g + 1], x[3 * g + 2]);
  l1[5] = max3f(x[15], y[0], y[1]);
#pragma unroll
  for (int g = 0; g < 4; ++g) l1[6 + g] = max3f(y[2 + 3 * g], y[3 + 3 * g], y[4 + 3 * g]);
  l1[10] = y[14];
  l1[11] = y[15];
  const float a = max3f(l1[0], l1[1], l1[2]), b = max3f(l1[3], l1[4], l1[5]);
  const float c = max3f(l1[6], l1[7], l1[8]), e = max3f(l1[9], l1[10], l1[11]);
  return fmaxf(max3f(a, b, c), e);
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
// (binary search; every index stays in [0, n_docs]; bounds clamped to
// [0, lim]). Without cu every position belongs to one document [0, lim).
struct DocBounds {
  int lo, hi;  // [lo, hi)
};
__device__ __forceinline__ DocBounds doc_bounds(const int32_t* cu, int n_docs, int i, int lim) {
  if (cu == nullptr) return {0, lim};
  int a = 0, b = n_docs - 1;  // find largest k in [0, n_docs-1] with cu[k] <= i
  while (a < b) {
    int m = (a + b + 1) >> 1;
    if (cu[m] <= i) a = m; else b = m - 1;
  }
  int lo = cu[a], hi = cu[a + 1];
  lo = lo < 0 ? 0 : (lo > lim ? lim : lo);
  hi = hi < lo ? lo : (hi > lim ? lim : hi);
  return {lo, hi};
}

// Allowed keys of local row r: the contiguous range [lo, hi] of local key
// indices (hi < lo when empty). Both ends are nondecreasing in r.
struct KeyRange {
  int lo, hi;
};
__device__ __forceinline__ KeyRange row_keys(const MaskGeom& m, int r) {
  const int gi = m.q_off + r;
  const DocBounds b = doc_bounds(m.cu, m.n_docs, gi, m.lim);
  const int lo = max(b.lo - m.k_off, 0);
  const int hi = m.causal ? min(gi - m.k_off, m.s_kv - 1) : min(b.hi - m.k_off, m.s_kv) - 1;
  return {lo, hi};
}

// Local query rows [lo, hi) that may see local key c (ignoring c < s_kv);
// lo may be negative, hi <= s_q. Both ends are nondecreasing in c.
struct RowSpan {
  int lo, hi;
};
__device__ __forceinline__ RowSpan key_rows(const MaskGeom& m, int c) {
  const int gj = m.k_off + c;
  const DocBounds b = doc_bounds(m.cu, m.n_docs, gj, m.lim);
  return {max(b.lo, m.causal ? gj : 0) - m.q_off, min(b.hi - m.q_off, m.s_q)};
}

// Entry b of a block order table (see block_order_launch), read through the
// scalar cache: the table is not written while a kernel that reads it runs,
// and b is wave-uniform.
__device__ __forceinline__ int order_entry(const int* order, int b) {
  typedef __attribute__((address_space(4))) const int* ConstInt;
  return ((ConstInt)(uintptr_t)order)[__builtin_amdgcn_readfirstlane(b)];
}

// Key-major workspace row length: padded so every 64-key tile is in bounds.
__host__ __device__ __forceinline__ int64_t kmajor_len(int64_t s_pad) {
  return (s_pad + 127) / 128 * 128;
}

}  // namespace usp
