// Pad + pack (sequence-sharded -> head-sharded) and unpack, for gfx950.
//
// The Ulysses exchange regroups every token's row [H][d] into P runs of
// hp = H/P heads, run r going to rank r ("feat(dspark): add Ulysses sequence
// parallel training", Modifications: shard and pad, separate Q/K/V
// all-to-alls). On one device that is a pure copy:
//     pack:   Y[r][s][:] = X[s][r*hp*d : (r+1)*hp*d]   (zero for s >= s_real)
//     unpack: X[s][r*hp*d : (r+1)*hp*d] = Y[r][s][:]
// It is HBM-bound with zero arithmetic, so the kernel is built around the
// memory system rather than the ALUs:
//   * the flat index t walks the token-major tensor X in order, so every
//     access to X is perfectly coalesced and every run of Y (hp*d elements,
//     256 B .. 4 KiB here) is written or read contiguously;
//   * 16-byte chunks per lane. The unpack keeps 3 independent chunks in
//     flight per lane (all loads issued before the stores) to cover HBM
//     latency; the pack, whose stores scatter into P runs, runs one chunk per
//     lane in more workgroups (measured: 6.38 TB/s against 5.90 with 4; the
//     unpack measured best at 3 of 2, 3, 4, 6, 8);
//   * non-temporal loads and stores: nothing is reused, so the copy streams
//     past the caches instead of evicting the attention working set;
//   * integer division by the run and row lengths uses a multiply-high
//     reciprocal computed once on the host, keeping the VALU cost per chunk a
//     few instructions.
#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

template <typename Chunk, bool kPack, int kUnroll>
__global__ __launch_bounds__(256) void permute_kernel(const Chunk* __restrict__ src,
                                                      Chunk* __restrict__ dst, uint32_t total,
                                                      uint32_t s_real, uint32_t s_pad,
                                                      FastDiv row_chunks, FastDiv run_chunks) {
  const uint32_t base = blockIdx.x * (256u * kUnroll) + threadIdx.x;
  Chunk val[kUnroll];
  uint32_t yidx[kUnroll];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t t = base + u * 256u;
    live[u] = t < total;
    uint32_t s = row_chunks.div(t);
    uint32_t c = t - s * row_chunks.d;
    uint32_t r = run_chunks.div(c);
    uint32_t off = c - r * run_chunks.d;
    yidx[u] = (r * s_pad + s) * run_chunks.d + off;
    if constexpr (kPack) {
      if (live[u] && s < s_real) {
        val[u] = __builtin_nontemporal_load(src + t);
      } else {
        val[u] = Chunk{};
      }
    } else {
      if (live[u]) val[u] = __builtin_nontemporal_load(src + yidx[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t t = base + u * 256u;
    if (!live[u]) continue;
    if constexpr (kPack) {
      __builtin_nontemporal_store(val[u], dst + yidx[u]);
    } else {
      __builtin_nontemporal_store(val[u], dst + t);
    }
  }
}

template <typename Chunk, bool kPack>
int launch(const void* src, void* dst, int64_t s_real, int64_t s_pad, int64_t row_bytes,
           int64_t run_bytes, hipStream_t stream) {
  constexpr int kUnroll = kPack ? 1 : 3;
  const int64_t rows = kPack ? s_pad : s_real;
  const int64_t row_chunks = row_bytes / (int64_t)sizeof(Chunk);
  const int64_t run_chunks = run_bytes / (int64_t)sizeof(Chunk);
  const int64_t total = rows * row_chunks;
  if (total == 0) return USP_OK;
  const int64_t per_block = 256 * kUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  TraceScope ts(kPack ? "pack_seq2head" : "unpack_head2seq", stream);
  hipLaunchKernelGGL((permute_kernel<Chunk, kPack, kUnroll>), dim3((unsigned)blocks), dim3(256),
                     0, stream, static_cast<const Chunk*>(src), static_cast<Chunk*>(dst),
                     (uint32_t)total, (uint32_t)s_real, (uint32_t)s_pad,
                     FastDiv::make((uint32_t)row_chunks), FastDiv::make((uint32_t)run_chunks));
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

}  // namespace

int permute_launch(bool pack, const void* src, void* dst, int64_t s_real, int64_t s_pad,
                   int p, int64_t row_bytes, hipStream_t stream) {
  const int64_t run_bytes = row_bytes / p;
  // widest chunk that divides a run
  if (run_bytes % 16 == 0) {
    return pack ? launch<u32x4, true>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream)
                : launch<u32x4, false>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream);
  }
  if (run_bytes % 8 == 0) {
    return pack ? launch<u32x2, true>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream)
                : launch<u32x2, false>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream);
  }
  return pack ? launch<unsigned, true>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream)
              : launch<unsigned, false>(src, dst, s_real, s_pad, row_bytes, run_bytes, stream);
}

}  // namespace usp
