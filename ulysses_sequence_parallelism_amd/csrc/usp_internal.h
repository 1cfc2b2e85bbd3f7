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
  int64_t s_pad, s_valid;
  const int32_t* cu;
  int n_docs;
  int hq, hkv, d;
  float scale;
  int causal;
  hipStream_t stream;
};

int kmajor_launch(const void* src, void* dst, int64_t s_pad, int heads, int64_t s_t,
                  hipStream_t stream, const char* trace_name);

size_t attn_fwd_bf16_workspace(int64_t s_pad, int hq, int hkv, int d);
size_t attn_bwd_bf16_workspace(int64_t s_pad, int hq, int hkv, int d);
int attn_fwd_bf16(const AttnArgs& a);
int attn_bwd_bf16(const AttnArgs& a);
int attn_fwd_f32(const AttnArgs& a);
int attn_bwd_f32(const AttnArgs& a);
size_t attn_bwd_f32_workspace(int64_t s_pad, int hq, int hkv, int d);

}  // namespace usp
