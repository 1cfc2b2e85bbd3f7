// Internal declarations shared by the libusp translation units (not ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/usp.h"

namespace usp {

// Kernel tracing: brackets one launch with HIP events when tracing is enabled.
bool trace_on();
struct TraceScope {
  const char* name;
  hipStream_t s;
  hipEvent_t start;
  TraceScope(const char* n, hipStream_t st);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;
};

// Unsigned 32-bit division by an invariant divisor via a multiply-high
// reciprocal (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (umulhi(n, m) + n) >> l for every
// 32-bit n (the sum is formed in 64 bits).
struct FastDiv {
  uint32_t d, m, l;
  static FastDiv make(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t hi = __umulhi(n, m);
#else
    const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
    return (uint32_t)(((uint64_t)hi + n) >> l);
  }
};

int permute_launch(bool pack, const void* src, void* dst, int64_t s_real, int64_t s_pad, int p,
                   int64_t row_bytes, hipStream_t stream);

// One attention call. Query rows sit at global positions q_off + [0, s_q),
// keys at k_off + [0, s_k), of which the first s_kv are valid; lim is the
// global extent (documents are clamped to it). The full-sequence entry points
// use q_off = k_off = 0, s_q = s_k = lim = s_pad and s_kv = s_valid.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* o_out;
  float* lse_out;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  size_t workspace_bytes;
  int64_t s_q, s_k, s_kv, q_off, k_off, lim;
  const int32_t* cu;
  int n_docs;
  int hq, hkv, d;
  float scale;
  int causal;
  int out_f32;     // outputs (O, or dQ/dK/dV) are fp32 instead of bf16
  int accumulate;  // backward, fp32 outputs: add to the existing contents
  hipStream_t stream;
};

// Mask geometry on global positions, as the kernels see it. Query row r of a
// call sits at global position q_off + r, key c at k_off + c; key c is allowed
// for row r iff c < s_kv, both positions lie in one document and, when causal,
// the key's position does not exceed the row's.
struct MaskGeom {
  const int32_t* cu;
  int n_docs, lim;     // documents, position clamp (global extent)
  int q_off, k_off;    // global position of local row 0 / key 0
  int s_q, s_k, s_kv;  // query rows, key rows, valid key rows
  int causal;
};

inline MaskGeom mask_geom(const AttnArgs& a) {
  MaskGeom m{};
  m.cu = a.cu;
  m.n_docs = a.n_docs;
  m.lim = (int)a.lim;
  m.q_off = (int)a.q_off;
  m.k_off = (int)a.k_off;
  m.s_q = (int)a.s_q;
  m.s_k = (int)a.s_k;
  m.s_kv = (int)a.s_kv;
  m.causal = a.causal;
  return m;
}

// Key-major copy of a [s_pad][heads][d] bf16 tensor (d = 128 or 64) into
// [heads][d][s_t], reordered within 16-position chunks (kmajor.hip).
int kmajor_launch(const void* src, void* dst, int64_t s_pad, int heads, int d, int64_t s_t,
                  hipStream_t stream, const char* trace_name);

// Key splits of a query-stationary kernel (splits.hip): query blocks of qrows
// rows over keys in tiles of key_tile, heads workgroups per block, slots
// workgroups resident at once; at most cap splits of at least min_tiles tiles.
// The combining kernel moves item_bytes per (block, split) it reads and
// fixed_bytes once; tile_bytes is that traffic's worth in one tile-time of one
// workgroup.
struct SplitProblem {
  int64_t s_q, q_off, k_off, s_kv;
  int causal;
  int qrows, heads, key_tile;
  int slots, cap, min_tiles;
  double item_bytes, fixed_bytes, tile_bytes;
};
struct SplitPlan {
  int n_split, split_tiles;  // splits (1: none) and tiles per split
};
SplitPlan plan_key_splits(const SplitProblem& p);

// Longest-first order of a grid's blocks for calls with packed documents
// (splits.hip): kind kOrderQueryBlocks (blocks of `block` query rows over key
// tiles of `tile`) or kOrderKeyBlocks (blocks of `block` keys over row tiles of
// `tile`). Needs block_order_bytes(n) bytes of device memory at `room`; on
// success *order points into it (n block indexes, longest first), or is NULL
// (the natural order) for more than 131,072 blocks.
enum { kOrderQueryBlocks = 0, kOrderKeyBlocks = 1 };
size_t block_order_bytes(int64_t n);
int block_order_launch(const MaskGeom& m, int kind, int n, int block, int tile, void* room,
                       hipStream_t stream, const int** order);

size_t attn_fwd_bf16_workspace(int64_t s_k, int hq, int hkv, int d);
size_t attn_fwd_bf16_min_workspace(int64_t s_k, int hkv, int d);  // the V copy alone
size_t attn_bwd_bf16_workspace(int64_t s_q, int64_t s_k, int hq, int hkv, int d);
// the part without room for dQ key splits
size_t attn_bwd_bf16_min_workspace(int64_t s_q, int64_t s_k, int hq, int hkv, int d);
// Key splits the bf16 dQ kernel runs for these arguments (1: a single pass).
int attn_bwd_bf16_dq_splits(const AttnArgs& a);
int attn_fwd_bf16(const AttnArgs& a);
// Key splits the bf16 forward runs for these arguments (1: a single pass).
int attn_fwd_bf16_splits(const AttnArgs& a);
int attn_bwd_bf16(const AttnArgs& a);
int attn_fwd_f32(const AttnArgs& a);
int attn_bwd_f32(const AttnArgs& a);
size_t attn_bwd_f32_workspace(int64_t s_q, int hq, int hkv, int d);
int attn_merge_launch(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                      void* o, float* lse, int64_t s_q, int hq, int d, int out_f32,
                      hipStream_t stream);

}  // namespace usp
