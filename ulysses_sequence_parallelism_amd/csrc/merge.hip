// Exact merge of two partial attention results over disjoint key sets.
//
// Ring / USP attention computes, per ring step, the attention of the local
// query rows against one block of keys, giving a partial output O_r (each row
// normalised over that block only) and its natural-log LSE_r; USP runs such
// ring steps inside the Ulysses head groups ("feat(dspark): add Ulysses
// sequence parallel training", Accuracy Test, Ulysses x Ring degrees;
// "[trainer] feat: support sequence parallel", review overview, the
// (dp, ring, ulysses) mesh). The softmax over the union of two key sets is
//     LSE = log(exp(LSE_a) + exp(LSE_b))
//     O   = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b
// which this kernel evaluates as m = max(LSE_a, LSE_b),
// LSE = m + log1p(exp(min - m)), so no exponential overflows; a row whose two
// LSEs are both -inf (no allowed key yet) stays O = 0, LSE = -inf.
//
// Memory-bound elementwise work: each thread owns 4 consecutive fp32 values of
// one (row, head) and the (row, head) groups never straddle a wavefront, so an
// in-place call (output = input a) reads every value before it is replaced.
#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb,
                                              float& lse) {
  const float m = fmaxf(la, lb);
  if (m == -INFINITY) {
    wa = wb = 0.f;
    lse = -INFINITY;
    return;
  }
  const float ea = expf(la - m), eb = expf(lb - m);  // one of them is exactly 1
  const float inv = 1.f / (ea + eb);
  wa = ea * inv;
  wb = eb * inv;
  lse = m + log1pf(fminf(ea, eb));
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* o_a, const float* lse_a,
                                                    const float* o_b, const float* lse_b,
                                                    void* o, float* lse, int s_q, FastDiv hq,
                                                    int n, int out_f32) {
  constexpr int C = D / 4;  // threads per (row, head)
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int rh = t / C, c = t % C;
  const uint32_t i = hq.div((uint32_t)rh);
  const int h = rh - (int)(i * hq.d);
  const int64_t li = (int64_t)h * s_q + i;
  float wa, wb, l;
  merge_weights(lse_a[li], lse_b[li], wa, wb, l);
  const int64_t e = (int64_t)rh * D + c * 4;
  const f32x4 a = *reinterpret_cast<const f32x4*>(o_a + e);
  const f32x4 b = *reinterpret_cast<const f32x4*>(o_b + e);
  const f32x4 r = a * wa + b * wb;
  if (out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + e) = r;
  } else {
    u32x2 v2 = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(o) + e) = v2;
  }
  if (c == 0) lse[li] = l;
}

}  // namespace

int attn_merge_launch(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                      void* o, float* lse, int64_t s_q, int hq, int d, int out_f32,
                      hipStream_t stream) {
  const int n = (int)(s_q * hq * (d / 4));
  const dim3 grid((unsigned)((n + 255) / 256));
  TraceScope ts("attn_merge", stream);
  const FastDiv fd = FastDiv::make((uint32_t)hq);
  if (d == 64)
    hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(256), 0, stream, o_a, lse_a, o_b, lse_b, o,
                       lse, (int)s_q, fd, n, out_f32);
  else
    hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(256), 0, stream, o_a, lse_a, o_b, lse_b, o,
                       lse, (int)s_q, fd, n, out_f32);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

}  // namespace usp
