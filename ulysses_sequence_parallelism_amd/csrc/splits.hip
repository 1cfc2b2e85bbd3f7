// Host-side planning of key splits for the query-stationary kernels (the
// attention forward and dQ).
//
// Such a kernel gives each workgroup a block of query rows and walks every
// key tile those rows may see. On a short sequence the grid is too small to
// fill the chip, and under a causal mask the last query blocks walk many times
// more tiles than the first. A split cuts each block's tile range into up to
// `cap` consecutive pieces run by separate workgroups, which write partial
// results that a second kernel combines; the plan picks the count that
// minimises the estimated time.
#include <algorithm>
#include <queue>
#include <vector>

#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

SplitPlan plan_key_splits(const SplitProblem& p) {
  if (p.cap <= 1 || p.s_q < 1) return {1, 0};
  // tiles per query block without documents (which only shorten a block's
  // range): the block's first row sees key 0 onwards, its last row up to
  // its causal limit
  const int nqb = (int)((p.s_q + p.qrows - 1) / p.qrows);
  std::vector<int> nt(nqb);
  int max_nt = 0;
  for (int b = 0; b < nqb; ++b) {
    const int64_t last = std::min<int64_t>((int64_t)(b + 1) * p.qrows, p.s_q) - 1;
    const int64_t hi = p.causal ? std::min(p.q_off + last - p.k_off, p.s_kv - 1) : p.s_kv - 1;
    nt[b] = hi >= 0 ? (int)(hi / p.key_tile + 1) : 0;
    max_nt = std::max(max_nt, nt[b]);
  }
  // Each candidate is scored by simulating the hardware's dispatch of the
  // grid, in tile-times of one workgroup: workgroups go round-robin to the
  // kXcds dies by linear index, and each die hands its next workgroup to the
  // first of its slots that frees. The grid runs query blocks heaviest first,
  // a block's splits adjacent in the order the kernels use: k for an odd Z,
  // (k + block) mod Z for an even one, so that no die receives only the
  // first (full) piece of every block. The combining kernel's traffic is
  // added in the same unit. Splitting must save 15%.
  constexpr int kXcds = 8;
  double base = 0, best_cost = 0;
  SplitPlan best{1, 0};
  for (int z = 1; z <= p.cap; ++z) {
    const int c = (max_nt + z - 1) / z;
    if (z > 1 && c < p.min_tiles) break;
    std::vector<std::priority_queue<double, std::vector<double>, std::greater<double>>> free_at(
        kXcds);
    for (int x = 0; x < kXcds; ++x)
      for (int i = 0; i < p.slots / kXcds; ++i) free_at[x].push(0.0);
    double makespan = 0, items = 0;
    int64_t idx = 0;
    for (int y = 0; y < p.heads; ++y)
      for (int b = nqb - 1; b >= 0; --b)
        for (int k = 0; k < z; ++k, ++idx) {
          const int piece = (z & 1) ? k : (k + b) % z;
          const int len = z > 1 ? std::min(nt[b] - piece * c, c) : nt[b];
          if (len <= 0) continue;
          auto& q = free_at[idx % kXcds];
          const double f = q.top() + len + 0.5;  // 0.5: prologue and epilogue
          q.pop();
          q.push(f);
          makespan = std::max(makespan, f);
          items += 1;
        }
    double cost = makespan;
    if (z > 1) cost += 2.0 + (items * p.item_bytes + p.fixed_bytes) / p.tile_bytes;
    if (z == 1) {
      base = best_cost = cost;
    } else if (cost < 0.85 * base && cost < best_cost) {
      best_cost = cost;
      best = {z, c};
    }
  }
  return best;
}

// ---------------------------------------------------------------------------
// Longest-first block order for calls with packed documents. Without
// documents the grids already run their blocks longest-first (the causal
// triangle's work grows with the query block and shrinks with the key block);
// with documents every document is its own triangle, so that order
// interleaves long and short blocks. These two kernels give a permutation of
// the blocks by decreasing work, ties by block index (the plan is
// deterministic); the attention kernels then map workgroup b to block
// order[b]. The order only schedules: every block's arithmetic is unchanged.

namespace {

// Work of each block in tiles: query blocks of `block` rows walk the key tiles
// of `tile` keys from the tile of their first row's first key to their last
// row's last key (the forward and dQ tile ranges); key blocks of `block` keys
// walk the row tiles of `tile` rows from their first key's first row to their
// last key's last row (the dK/dV range), none past the valid keys. Also
// clears the rank counts.
__global__ __launch_bounds__(256) void block_cost_kernel(MaskGeom m, int kind, int n, int block,
                                                         int tile, int* __restrict__ cost,
                                                         int* __restrict__ rank) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= n) return;
  int c = 0;
  if (kind == kOrderQueryBlocks) {
    const int q0 = b * block, q1 = min(q0 + block, m.s_q);
    const KeyRange kf = row_keys(m, q0), kl = row_keys(m, q1 - 1);
    const int t0 = kf.lo / tile * tile;
    c = kl.hi >= kf.lo ? (kl.hi - t0) / tile + 1 : 0;
  } else {
    const int j0 = b * block, j1 = min(j0 + block, m.s_k);
    const RowSpan rf = key_rows(m, j0), rl = key_rows(m, j1 - 1);
    const int rstart = max(rf.lo, 0), rend = rl.hi - 1;
    c = (j0 < m.s_kv && rend >= rstart) ? rend / tile - rstart / tile + 1 : 0;
  }
  cost[b] = c;
  rank[b] = 0;
}

// rank(i) = #{j : cost_j > cost_i} + #{j < i : cost_j = cost_i}, counted over
// j in chunks of 256 (grid y) held in LDS and read 4 at a time; the chunk
// counts are added with integer atomics (a sum: the result does not depend on
// their order).
__global__ __launch_bounds__(256) void block_rank_kernel(const int* __restrict__ cost, int n,
                                                         int* __restrict__ rank) {
  __shared__ __attribute__((aligned(16))) int chunk[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int j0 = blockIdx.y * 256;
  // past the end: a cost no block has (-1), never counted
  chunk[threadIdx.x] = j0 + (int)threadIdx.x < n ? cost[j0 + threadIdx.x] : -1;
  __syncthreads();
  if (i >= n) return;
  const int ci = cost[i];
  const int rel = i - j0;  // chunk positions below rel precede i
  int r = 0;
#pragma unroll 8
  for (int t = 0; t < 256; t += 4) {
    const int4 c4 = *reinterpret_cast<const int4*>(&chunk[t]);
    r += (c4.x > ci || (c4.x == ci && t < rel)) ? 1 : 0;
    r += (c4.y > ci || (c4.y == ci && t + 1 < rel)) ? 1 : 0;
    r += (c4.z > ci || (c4.z == ci && t + 2 < rel)) ? 1 : 0;
    r += (c4.w > ci || (c4.w == ci && t + 3 < rel)) ? 1 : 0;
  }
  if (r != 0) atomicAdd(&rank[i], r);
}

// order[rank(i)] = i: the ranks are a permutation of [0, n).
__global__ __launch_bounds__(256) void block_scatter_kernel(const int* __restrict__ rank, int n,
                                                            int* __restrict__ order) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) order[rank[i]] = i;
}

}  // namespace

size_t block_order_bytes(int64_t n) { return (size_t)((n * 4 + 255) / 256 * 256) * 3; }

constexpr int kMaxOrderBlocks = 131072;

int block_order_launch(const MaskGeom& m, int kind, int n, int block, int tile, void* room,
                       hipStream_t stream, const int** order) {
  // The rank kernel's work grows with n^2 and its grid is (n/256)^2
  // workgroups: past 131,072 blocks (8.4M rows at 64 per block) the call keeps
  // the natural order, which gives the same results.
  if (n < 1 || n > kMaxOrderBlocks) {
    *order = nullptr;
    return USP_OK;
  }
  const size_t part = block_order_bytes(n) / 3;
  int* cost = static_cast<int*>(room);
  int* rank = reinterpret_cast<int*>(static_cast<char*>(room) + part);
  int* ord = reinterpret_cast<int*>(static_cast<char*>(room) + 2 * part);
  const unsigned nb = (unsigned)((n + 255) / 256);
  TraceScope ts("attn_block_order", stream);
  hipLaunchKernelGGL(block_cost_kernel, dim3(nb), dim3(256), 0, stream, m, kind, n, block, tile,
                     cost, rank);
  if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
  hipLaunchKernelGGL(block_rank_kernel, dim3(nb, nb), dim3(256), 0, stream, cost, n, rank);
  if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
  hipLaunchKernelGGL(block_scatter_kernel, dim3(nb), dim3(256), 0, stream, rank, n, ord);
  if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
  *order = ord;
  return USP_OK;
}

}  // namespace usp
