// Key-major (transposed) copies of a [s_pad][H][d] bf16 tensor (d = 128 or 64)
// for gfx950.
//
// In the attention kernels the matrix-core reduction axis of P.V (forward),
// of dS.K (dQ) and of P^T.dO, dS^T.Q (dK/dV) is the sequence axis. A 32x32x16
// MFMA operand wants 8 consecutive reduction elements per lane, so the
// operand that is row-major in the sequence ([s][H][d]) is staged from a
// copy laid out [H][d][s] instead. Inside each 16-element chunk of s the copy
// stores position p at slot kperm(p) (bits 2 and 3 swapped), which matches the
// order in which a lane holds the other operand straight out of a 32x32
// accumulator, so both operands are read with single 16-byte loads.
// Slots at and beyond s_pad are written as zero.
//
// One block transposes a 64-position x d-column tile of one head through LDS:
// 16-byte coalesced loads from the row-major tensor, then every lane gathers 8
// positions of one column and writes one 16-byte chunk.
#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

constexpr int T = 64;

template <int D>
__global__ __launch_bounds__(256) void kmajor_kernel(const unsigned short* __restrict__ src,
                                                     unsigned short* __restrict__ dst,
                                                     int s_pad, int heads, int64_t s_t) {
  constexpr int P = D + 8;   // LDS row pitch (elements)
  constexpr int KC = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) unsigned short tile[T * P];
  const int h = blockIdx.y;
  const int s0 = blockIdx.x * T;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < T * KC / 256; ++u) {
    const int e = tid + 256 * u;
    const int r = e / KC, c = e % KC;
    const int s = s0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (s < s_pad) val = *reinterpret_cast<const u32x4*>(src + ((int64_t)s * heads + h) * D + c * 8);
    *reinterpret_cast<u32x4*>(&tile[r * P + c * 8]) = val;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < D * (T / 8) / 256; ++u) {
    const int e = tid + 256 * u;
    const int col = e >> 3, c8 = e & 7;  // output row (column of src), 8-slot chunk
    unsigned w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p0 = c8 * 8 + 2 * t;
      const int l0 = (p0 & ~15) | kperm(p0 & 15);
      const int l1 = ((p0 + 1) & ~15) | kperm((p0 + 1) & 15);
      w[t] = (unsigned)tile[l0 * P + col] | ((unsigned)tile[l1 * P + col] << 16);
    }
    u32x4 out = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(dst + ((int64_t)h * D + col) * s_t + s0 + c8 * 8) = out;
  }
}

}  // namespace

int kmajor_launch(const void* src, void* dst, int64_t s_pad, int heads, int d, int64_t s_t,
                  hipStream_t stream, const char* trace_name) {
  dim3 grid((unsigned)(s_t / T), (unsigned)heads);
  TraceScope ts(trace_name, stream);
  auto* s = static_cast<const unsigned short*>(src);
  auto* o = static_cast<unsigned short*>(dst);
  if (d == 64)
    hipLaunchKernelGGL(kmajor_kernel<64>, grid, dim3(256), 0, stream, s, o, (int)s_pad, heads, s_t);
  else
    hipLaunchKernelGGL(kmajor_kernel<128>, grid, dim3(256), 0, stream, s, o, (int)s_pad, heads, s_t);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

}  // namespace usp
