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

}  // namespace usp
