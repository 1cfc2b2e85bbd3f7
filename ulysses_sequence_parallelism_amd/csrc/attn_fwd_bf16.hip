// Attention forward, bf16 in / fp32 accumulate, d = 128 or 64, gfx950 matrix cores.
//
// One rank's share of Ulysses attention is exact softmax attention over the
// whole sequence for hq query heads sharing hkv key/value heads ("feat(dspark):
// add Ulysses sequence parallel training", Modifications: local attention after
// the Q/K/V all-to-alls, Q and KV head counts handled separately). Query row i
// may use key j iff j < s_valid, doc(j) == doc(i) and j <= i when causal
// (packed documents: "GLM-5.2 131k context parallelism", Purpose). The kernel
// returns O and the natural-log LSE of every row.
//
// The same kernel serves a query interval against a key interval on global
// positions (rows at q_off + i, keys at k_off + j, the causal test and the
// documents taken on those positions): the partial (O, LSE) of one ring step
// of Ring / USP attention, merged exactly afterwards (the ring degree of USP:
// "feat(dspark)", Accuracy Test; "[trainer] feat: support sequence parallel",
// review overview, the (dp, ring, ulysses) mesh), and a contiguous
// context-parallel rank's query rows against the whole sequence with a causal
// offset and global document offsets ("GLM-5.2 131k context parallelism",
// Purpose). O may be written in fp32 for the merge.
//
// Design (gfx950):
//   * Workgroup = 8 waves that share one KV head: HG query heads of the group
//     times 8/HG blocks of 32 query rows. Each staged K/V tile feeds every
//     wave, so a K/V byte brought into LDS serves 8*32 query rows.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     a lane then owns ONE query row (column l%32) and 16 keys per 32-key
//     block, so the softmax row max / row sum are in-lane reductions plus one
//     v_permlane32_swap across the two half-waves, and the row statistics
//     (running max, sum, mask bounds) are per-lane scalars.
//   * The probabilities go straight from the accumulator into the B operand of
//     O^T += V^T P^T (no LDS round trip); V is staged from a key-major copy
//     whose 16-key chunks are reordered to match (see kmajor.hip).
//   * Q stays in registers for the whole key loop (d / 16 x 16 bytes per lane).
//   * K and V^T tiles of 64 keys sit in three LDS slots each and go straight
//     from global memory into LDS (global_load_lds_dwordx4: no staging
//     registers, no LDS stores). That load writes each lane's 16 bytes at
//     consecutive LDS addresses, so rows are unpadded and their 16-byte chunks
//     XOR-swizzled (chunk c of a K row r in slot c ^ swz_row(r), of a 128-byte
//     V^T row r in slot c ^ ((r >> 1) & 7)): 16 lanes reading one chunk of 16
//     rows hit 16 distinct bank groups.
//   * Ping-pong between the two waves of each SIMD: every tile has a softmax
//     phase (row max, exponentials, row sums: vector work) and a matrix phase
//     (the next tile's scores and this tile's P V: MFMA). The waves of one
//     half of the workgroup run half a tile behind the other half, with a
//     barrier between phases, so on every SIMD one wave feeds the matrix core
//     while its partner does the vector work. Boundary tiles and running-max
//     updates take a rarely used slow path inside the softmax phase.
//   * Online softmax in the log2 domain (scale*log2(e) folded into one FMA
//     before v_exp_f32) with a lazy, exact rescale: the running max is only
//     raised when a row's tile max exceeds it by more than 8 (log2 units), so
//     probabilities stay <= 2^8 and the O rescale is skipped on almost every
//     tile; the final normalisation uses the same running max, so nothing is
//     approximated.
//   * Causal / document / padding masks are applied only on tiles that cross
//     a boundary; tiles entirely outside every row's range are never visited.
//   * Workgroups are launched heaviest-first (last query block first) so the
//     causal triangle's long rows start early and the tail is short. With
//     packed documents that order interleaves long and short blocks, so a
//     one-pass call takes a longest-first order computed on the device from
//     the documents (splits.hip), which changes only the schedule.
//   * Short sequences (a grid of a few hundred workgroups) split each query
//     block's key tiles into consecutive pieces run by separate workgroups
//     (planned in splits.hip); each writes an fp32 partial O and its LSE, and
//     a merge kernel combines them exactly, as the merge of ring steps does.
#include <algorithm>
#include <type_traits>

#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

constexpr int BN = 64;        // keys per tile
constexpr float kRescaleThreshold = 8.0f;

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* vt;   // key-major V: [hkv][D][s_t], 16-chunk reordered
  __bf16* o;          // [s_q][hq][D], or NULL when o32 is set
  float* o32;         // fp32 O instead of bf16 (NULL otherwise)
  float* lse;         // [hq][s_q]
  MaskGeom m;
  int64_t s_t;
  int hq, hkv, n_qblocks;
  float scale_log2;   // softmax scale * log2(e)
  // Key splits: with n_split > 1 the workgroups of one query block share its
  // tile range, split z taking tiles [z, z + 1) * split_tiles of it, and write
  // fp32 partial O / LSE at o32 + z * o_split and lse + z * lse_split.
  int n_split, split_tiles;
  int64_t o_split, lse_split;
  // longest-first order of the query blocks (calls with packed documents), or
  // NULL: the natural order, last block first
  const int* order;
};

template <int D, int HG>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdParams pr) {
  constexpr int KK = D / 16;     // 16-wide reduction steps of Q K^T
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int KC = D / 8;      // 16-byte chunks per K row
  constexpr int RPP = 64 / KC;   // K rows per 1 KiB wave-load
  constexpr int KPW = BN / RPP / 8;  // K wave-loads per wave and tile
  constexpr int VPW = D / 8 / 8;     // V^T wave-loads (8 d-rows each) per wave and tile
  constexpr int QBW = 8 / HG;
  constexpr int QROWS = 32 * QBW;
  // three slots per tensor in one array each, slot s sitting s tiles after
  // slot 0 (the fragment reads below add that as a constant)
  __shared__ __attribute__((aligned(16))) __bf16 lk[3][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 lv[3][D * BN];
  // filled only by direct loads, which this compiler does not count as stores
  asm volatile("" ::"s"(&lk[0][0]), "s"(&lv[0][0]) : "memory");
  auto kslot = [&](int b) -> __bf16* { return &lk[b][0]; };
  auto vslot = [&](int b) -> __bf16* { return &lv[b][0]; };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, ln = lane & 31;
  const int g = pr.hq / pr.hkv;
  const int chunks = g / HG;
  const int kvh = blockIdx.y / chunks, hc = blockIdx.y % chunks;
  const int head = kvh * g + hc * HG + (w % HG);
  // heaviest query block first; its key splits follow one another. With an
  // even count the order is rotated by the block, so that the round-robin
  // over the 8 dies does not send every block's first piece to the same dies
  // (an odd count is coprime with 8 and keeps the full pieces first).
  const int bi = (int)blockIdx.x / pr.n_split;
  const int qb = pr.order ? order_entry(pr.order, bi) : pr.n_qblocks - 1 - bi;
  const int zk = (int)blockIdx.x % pr.n_split;
  const int zs = (pr.n_split & 1) ? zk : (zk + qb) % pr.n_split;
  const int q0 = qb * QROWS;
  const int s_q = pr.m.s_q, s_k = pr.m.s_k;
  const int q1 = min(q0 + QROWS, s_q);
  const int wq0 = q0 + (w / HG) * 32;
  const int qi = wq0 + ln;
  const bool row_ok = qi < s_q;
  const int qc = row_ok ? qi : s_q - 1;

  // this lane's allowed keys [lo, hi]
  const KeyRange kr = row_keys(pr.m, qc);
  const int lo = kr.lo, hi = kr.hi;
  // workgroup key range and the range that needs no mask (both ends of a
  // row's range are nondecreasing in the row)
  const KeyRange kfirst = row_keys(pr.m, q0), klast = row_keys(pr.m, q1 - 1);
  // with key splits, the part of it in this split's tiles (tiles counted from
  // the one holding the first key, as without splits)
  const int t_split = (kfirst.lo / BN + zs * pr.split_tiles) * BN;
  const int kmin = pr.n_split > 1 ? max(kfirst.lo, t_split) : kfirst.lo;
  const int kmax = pr.n_split > 1 ? min(klast.hi, t_split + pr.split_tiles * BN - 1) : klast.hi;
  const int free_lo = klast.lo, free_hi = kfirst.hi;
  // this wave's key range (waves of one workgroup may cover different rows)
  const int wkmin = row_keys(pr.m, min(wq0, s_q - 1)).lo;
  const int wkmax = row_keys(pr.m, min(wq0 + 31, s_q - 1)).hi;

  // Q fragment: B operand of S^T = K Q^T, lane holds Q[qc][16kk + 8hl .. +7]
  bf16x8 qreg[KK];
  {
    const __bf16* qp = pr.q + ((int64_t)qc * pr.hq + head) * D + hl * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
  }
  // Retire the Q loads here; otherwise the wait-count pass treats them as
  // possibly in flight inside the loop and makes the MFMAs wait for the next
  // tile's loads too.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int tstart = (kmin / BN) * BN;
  const int nt = kmax >= kmin ? (kmax - tstart) / BN + 1 : 0;
  float* const o32 = pr.n_split > 1 ? pr.o32 + zs * pr.o_split : pr.o32;
  float* const lse_out = pr.n_split > 1 ? pr.lse + zs * pr.lse_split : pr.lse;
  if (pr.n_split > 1 && nt == 0) {  // nothing in this split: LSE = -inf tells the merge to skip it
    if (row_ok && hl == 0) lse_out[(int64_t)head * s_q + qi] = -INFINITY;
    return;
  }

  // Tile loads. A part is one 1 KiB wave-load: RPP keys of K or 8 d-rows of V^T. Wave w
  // loads K parts KPW w .. +KPW-1 and V^T parts VPW w .. +VPW-1 as inline-asm
  // direct loads (lds_dma16): a wave-uniform base plus a 32-bit lane offset.
  const int wu = __builtin_amdgcn_readfirstlane(w);  // LDS destinations go to M0
  const uint32_t key_bytes = (uint32_t)pr.hkv * D * 2;
  const uint32_t vt_row_bytes = (uint32_t)pr.s_t * 2;
  auto load_k = [&](int t, int slot) {
    const int t0 = tstart + t * BN;
    const uint32_t dst = lds_addr(kslot(slot));
    const char* kb = reinterpret_cast<const char*>(pr.k) + (int64_t)kvh * (D * 2);
    const int q = lane / KC;  // key within the part; lane % KC is the LDS slot
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int part = KPW * wu + j;
      // keys past the end read the last key (always masked)
      const int first = min(t0 + RPP * part, s_k - 1);
      const uint32_t rel = (uint32_t)(min(t0 + RPP * part + q, s_k - 1) - first);
      const uint32_t off =
          rel * key_bytes + ((uint32_t)((lane % KC) ^ swz_row<D>(RPP * part + q)) << 4);
      lds_dma16(kb + (int64_t)first * key_bytes, off, dst + part * 1024);
    }
  };
  auto load_v = [&](int t, int slot) {
    const int t0 = tstart + t * BN;
    const uint32_t dst = lds_addr(vslot(slot));
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int part = VPW * wu + j;
      const char* b = reinterpret_cast<const char*>(pr.vt + ((int64_t)kvh * D + 8 * part) * pr.s_t + t0);
      // row 8 part + lane / 8 sits in slot chunk ^ ((row >> 1) & 7)
      const uint32_t off = (uint32_t)(lane >> 3) * vt_row_bytes +
                           ((uint32_t)((lane & 7) ^ (4 * (part & 1) + (lane >> 4))) << 4);
      lds_dma16(b, off, dst + part * 1024);
    }
  };
  // LDS byte addresses of the lane's fragments in slot 0 of each array, kept
  // opaque to the compiler: a read of slot s, block b is then one register
  // plus a constant in the read's 16-bit offset field. With element offsets
  // the compiler kept more address registers and spilled.
  uint32_t kra[KK], vra[4];
  {
    const uint32_t kb0 = lds_addr(&lk[0][0]), vb0 = lds_addr(&lv[0][0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kra[kk] = kb0 + 2 * (ln * D + (((hl + 2 * kk) ^ swz_row<D>(ln)) << 3));
      asm volatile("" : "+v"(kra[kk]));
    }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      vra[ch] = vb0 + 2 * (ln * BN + (((hl + 2 * ch) ^ ((ln >> 1) & 7)) << 3));
      asm volatile("" : "+v"(vra[ch]));
    }
  }
  // S^T = K Q^T for the two 32-key blocks of the tile in slot buf
  auto scores = [&](int buf, f32x16* sacc) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = lds_read_b128(kra[kk] + (uint32_t)(buf * BN * D + kb * 32 * D) * 2);
        sacc[kb] = mfma32(kf, qreg[kk], sacc[kb]);
      }
    }
  };

  // Two wave groups take turns: while the waves of one group run a tile's
  // matrix phase (the next tile's scores and this tile's P V, all MFMA), the
  // waves of the other run a softmax phase (row max, mask and rescale when
  // needed, exponentials, row sums: all vector work). Waves w and w + 4 share
  // a SIMD, so each SIMD holds one wave of each group and its matrix core is
  // fed by one while the other does the vector work. A barrier separates the
  // phases; the second group runs half a tile behind the first.
  // Tile t's K sits in K slot t % 3 and its V^T in V slot t % 3. The softmax
  // phase of tile t loads K(t+2) into the slot of K(t-1), and the matrix phase
  // of tile t loads V(t+1) into the slot of V(t-2); both were last read by the
  // matrix phase of tile t-2, which both groups have finished by then. The
  // other group's concurrent phase reads K(t+1) / V(t), K(t) / V(t-1) or no
  // LDS at all, never a slot being written. The matrix phase waits for all of
  // its wave's loads, so a tile's slots are complete at the barrier after both
  // groups' matrix phases of the tile before. (Splitting the loads this way
  // balances the two phases: all loads in the softmax phase, or all in the
  // matrix phase, measured slower.)
  const int grp = wu >> 2;
  f32x16 sc[2];   // scores of the tile whose softmax phase comes next
  bf16x8 pb[4];   // its probabilities, for the next matrix phase
  if (nt > 0) {
    load_k(0, 0);
    if (nt > 1) load_k(1, 1);
    load_v(0, 0);
  }
  wait_lds_dma();
  __syncthreads();
  if (nt > 0) scores(0, sc);

  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int t0 = tstart + t * BN;
    // -- row max of this tile (both half-waves hold the row); a full tile
    //    needs no mask
    float mx = half_swap_max(max_of_32(sc[0], sc[1])) * pr.scale_log2;
    // K(t+2) issued after the row max, not ahead of it (0.4% faster)
    if (t + 2 < nt) load_k(t + 2, (t + 2) % 3);
    const bool full = t0 >= free_lo && t0 + BN - 1 <= free_hi &&
                      t0 >= wkmin && t0 + BN - 1 <= wkmax;
    // -- slow path (boundary tiles and running-max updates, both rare): mask,
    //    recompute the max, rescale O
    if (__ballot(!full || mx > m_run + kRescaleThreshold)) {
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t0 + kb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
            if (key < lo || key > hi) sc[kb][i] = -INFINITY;
          }
        mx = half_swap_max(max_of_32(sc[0], sc[1])) * pr.scale_log2;
      }
      const bool need = mx > m_run + kRescaleThreshold;
      if (__ballot(need)) {
        const float mnew = need ? mx : m_run;
        const float alpha = need ? exp2f(m_run - mnew) : 1.f;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
        l_run *= alpha;
        m_run = mnew;
      }
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    float ls4[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 pk;
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][8 * c + 2 * u], pr.scale_log2, -msub));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][8 * c + 2 * u + 1], pr.scale_log2, -msub));
          ls += p0 + p1;
          pk[u] = pack_bf16x2(p0, p1);
        }
        ls4[kb * 2 + c] = ls;
        pb[kb * 2 + c] = __builtin_bit_cast(bf16x8, pk);
      }
    }
    l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
    // P and the row sum are complete here: without this the compiler may
    // sink the exponentials past the barrier into the matrix phase
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 u = __builtin_bit_cast(u32x4, pb[i]);
      asm volatile("" : "+v"(u));
      pb[i] = __builtin_bit_cast(bf16x8, u);
    }
    asm volatile("" : "+v"(l_run));
  };
  // matrix phase of tile t: K(t+1) in slot KS = (t+1) % 3, V(t) in VS = t % 3.
  // On the last tile K(t+1) does not exist and the scores are unused.
  auto matrix = [&](int t, auto ks, auto vs) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks)::value, VS = decltype(vs)::value;
    if (t + 1 < nt) load_v(t + 1, (t + 1) % 3);
    scores(KS, sc);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 vf = lds_read_b128(vra[ch] + (uint32_t)(VS * D * BN + b * 32 * BN) * 2);
        oacc[b] = mfma32(vf, pb[ch], oacc[b]);
      }
    }
    // fragment reads run four ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
    for (int i = 0; i < 2 * KK + 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    wait_lds_dma();  // this wave's K loads (softmax phase) and V loads (above) have landed
  };
  // The phases must not leak into each other: without a scheduling fence the
  // compiler moves register-only work (the exponentials) across a barrier.
  auto phase_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Every wave runs softmax(t), barrier, matrix(t), barrier for each tile.
  // The second group passes one barrier before its first tile and the first
  // group one after its last, so both pass the same number of barriers and the
  // second group's softmax phases meet the first group's matrix phases.
  auto tile = [&](int t, auto ks, auto vs) __attribute__((always_inline)) {
    softmax(t);
    phase_barrier();
    matrix(t, ks, vs);
    phase_barrier();
  };
  if (grp == 1) phase_barrier();
  int it = 0;
  for (; it + 3 <= nt; it += 3) {
    tile(it, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
    tile(it + 1, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
    tile(it + 2, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
  }
  if (it < nt) tile(it, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  if (it + 1 < nt) tile(it + 1, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  if (grp == 0) phase_barrier();

  const float l_tot = half_swap_sum(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t ob = ((int64_t)qi * pr.hq + head) * D + hl * 4;
    if (o32 != nullptr) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 v4 = {oacc[b][4 * r] * inv, oacc[b][4 * r + 1] * inv, oacc[b][4 * r + 2] * inv,
                      oacc[b][4 * r + 3] * inv};
          *reinterpret_cast<f32x4*>(o32 + ob + b * 32 + r * 8) = v4;
        }
    } else {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 v2 = {pack_bf16x2(oacc[b][4 * r] * inv, oacc[b][4 * r + 1] * inv),
                      pack_bf16x2(oacc[b][4 * r + 2] * inv, oacc[b][4 * r + 3] * inv)};
          *reinterpret_cast<u32x2*>(pr.o + ob + b * 32 + r * 8) = v2;
        }
    }
    if (hl == 0)
      lse_out[(int64_t)head * s_q + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Exact combination of the key splits of one call. Split z covered a disjoint
// range of key tiles and returned O_z normalised over its own keys and their
// natural-log LSE_z; over the union, with M = max_z LSE_z and
// w_z = exp(LSE_z - M),
//     O = sum_z w_z O_z / sum_z w_z,   LSE = M + log(sum_z w_z)
// (the same identity as the two-way merge of ring steps). A split whose LSE is
// -inf saw no allowed key of the row; its O is not read (an empty split never
// writes it). A row with no allowed key at all gets O = 0, LSE = -inf.
// Memory-bound: one thread per 8 consecutive values of one (row, head).
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* part, const float* plse,
                                                          int64_t o_split, int64_t lse_split,
                                                          int nz, void* o, float* lse, int s_q,
                                                          FastDiv hq, int n, int out_f32) {
  constexpr int C = D / 8;  // threads per (row, head)
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int rh = t / C, c = t % C;
  const uint32_t i = hq.div((uint32_t)rh);
  const int h = rh - (int)(i * hq.d);
  const int64_t li = (int64_t)h * s_q + i;
  float m = -INFINITY;
  for (int z = 0; z < nz; ++z) m = fmaxf(m, plse[z * lse_split + li]);
  const int64_t e = (int64_t)rh * D + c * 8;
  f32x4 a0 = {}, a1 = {};
  float l_out = -INFINITY;
  if (m != -INFINITY) {
    float ws = 0.f;
    for (int z = 0; z < nz; ++z) {
      const float lz = plse[z * lse_split + li];
      if (lz == -INFINITY) continue;
      const float wz = expf(lz - m);
      const float* pz = part + z * o_split + e;
      a0 += wz * *reinterpret_cast<const f32x4*>(pz);
      a1 += wz * *reinterpret_cast<const f32x4*>(pz + 4);
      ws += wz;
    }
    const float inv = 1.f / ws;  // ws >= 1: the split holding the maximum has weight 1
    a0 *= inv;
    a1 *= inv;
    l_out = m + logf(ws);
  }
  if (out_f32) {
    float* of = static_cast<float*>(o) + e;
    *reinterpret_cast<f32x4*>(of) = a0;
    *reinterpret_cast<f32x4*>(of + 4) = a1;
  } else {
    u32x4 v4 = {pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]), pack_bf16x2(a1[0], a1[1]),
                pack_bf16x2(a1[2], a1[3])};
    *reinterpret_cast<u32x4*>(static_cast<__bf16*>(o) + e) = v4;
  }
  if (c == 0) lse[li] = l_out;
}

int hg_for(int g) { return g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1; }

// Query rows per workgroup and workgroups of the unsplit grid.
int qrows_for(int hq, int hkv) { return 32 * (8 / hg_for(hq / hkv)); }
int64_t grid_size(int64_t s_q, int hq, int hkv) {
  const int g = hq / hkv;
  return (s_q + qrows_for(hq, hkv) - 1) / qrows_for(hq, hkv) * hkv * (g / hg_for(g));
}

// Key splits pay off only while the unsplit grid is short of a few rounds of
// workgroups on the 256 compute units (one 8-wave workgroup each).
constexpr int kCUs = 256;
constexpr int kMaxSplits = 8;
constexpr int kMinSplitTiles = 8;
int split_cap(int64_t s_q, int hq, int hkv) {
  const int64_t wgs = grid_size(s_q, hq, hkv);
  if (wgs >= 2 * kCUs) return 1;
  return (int)std::min<int64_t>(kMaxSplits, (4 * kCUs + wgs - 1) / wgs);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }
size_t vcopy_bytes(int64_t s_k, int hkv, int d) { return (size_t)hkv * d * kmajor_len(s_k) * 2; }
size_t split_bytes(int z, int64_t s_q, int hq, int d) {
  return z > 1 ? align256((size_t)z * s_q * hq * d * 4) + (size_t)z * hq * s_q * 4 : 0;
}

// Key splits of one call, within the workspace room for the partials. One
// tile of one 8-wave workgroup is 8 x 32 rows x 64 keys x 4d FLOP: at about
// 4.3 TFLOP/s per compute unit and 5 TB/s, d x 76 KB of traffic.
SplitPlan plan_splits(int64_t s_q, int64_t q_off, int64_t k_off, int64_t s_kv, int causal, int hq,
                      int hkv, int d, size_t room) {
  int cap = split_cap(s_q, hq, hkv);
  while (cap > 1 && split_bytes(cap, s_q, hq, d) > room) --cap;
  SplitProblem sp{};
  sp.s_q = s_q;
  sp.q_off = q_off;
  sp.k_off = k_off;
  sp.s_kv = s_kv;
  sp.causal = causal;
  sp.qrows = qrows_for(hq, hkv);
  sp.heads = (int)(grid_size(s_q, hq, hkv) / ((s_q + sp.qrows - 1) / sp.qrows));
  sp.key_tile = BN;
  sp.slots = kCUs;
  sp.cap = cap;
  sp.min_tiles = kMinSplitTiles;
  // each (block, split) partial O is written and read back; the final O written
  sp.item_bytes = (double)sp.qrows * hg_for(hq / hkv) * d * 8;
  sp.fixed_bytes = (double)s_q * hq * d * 2;
  sp.tile_bytes = 76.0e3 * d;
  return plan_key_splits(sp);
}

template <int D, int HG>
int launch_fwd(const FwdParams& p, int g, int hkv, hipStream_t stream) {
  constexpr int QROWS = 32 * (8 / HG);
  FwdParams pr = p;
  pr.n_qblocks = (p.m.s_q + QROWS - 1) / QROWS;
  dim3 grid((unsigned)(pr.n_qblocks * pr.n_split), (unsigned)(hkv * (g / HG)));
  TraceScope ts("attn_fwd_bf16", stream);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, HG>), grid, dim3(512), 0, stream, pr);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

template <int D>
int fwd_dispatch(const FwdParams& p, int g, int hkv, hipStream_t stream) {
  if (g % 4 == 0) return launch_fwd<D, 4>(p, g, hkv, stream);
  if (g % 2 == 0) return launch_fwd<D, 2>(p, g, hkv, stream);
  return launch_fwd<D, 1>(p, g, hkv, stream);
}

int split_merge_launch(const float* part, const float* plse, int64_t o_split, int64_t lse_split,
                       int nz, void* o, float* lse, int64_t s_q, int hq, int d, int out_f32,
                       hipStream_t stream) {
  const int n = (int)(s_q * hq * (d / 8));
  const dim3 grid((unsigned)((n + 255) / 256));
  TraceScope ts("attn_fwd_merge", stream);
  const FastDiv fd = FastDiv::make((uint32_t)hq);
  if (d == 64)
    hipLaunchKernelGGL((split_merge_kernel<64>), grid, dim3(256), 0, stream, part, plse, o_split,
                       lse_split, nz, o, lse, (int)s_q, fd, n, out_f32);
  else
    hipLaunchKernelGGL((split_merge_kernel<128>), grid, dim3(256), 0, stream, part, plse,
                       o_split, lse_split, nz, o, lse, (int)s_q, fd, n, out_f32);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

}  // namespace

// Bytes of the longest-first block order of s_q query rows.
static size_t fwd_order_bytes(int64_t s_q, int hq, int hkv) {
  return block_order_bytes((s_q + qrows_for(hq, hkv) - 1) / qrows_for(hq, hkv));
}

// The V copy, then room for the key splits of a call of s_k query rows, or for
// its block order (used only without splits).
size_t attn_fwd_bf16_workspace(int64_t s_k, int hq, int hkv, int d) {
  return vcopy_bytes(s_k, hkv, d) +
         std::max(split_bytes(split_cap(s_k, hq, hkv), s_k, hq, d), fwd_order_bytes(s_k, hq, hkv));
}

size_t attn_fwd_bf16_min_workspace(int64_t s_k, int hkv, int d) { return vcopy_bytes(s_k, hkv, d); }

int attn_fwd_bf16_splits(const AttnArgs& a) {
  const size_t v = vcopy_bytes(a.s_k, a.hkv, a.d);
  const size_t room = a.workspace_bytes > v ? a.workspace_bytes - v : 0;
  return plan_splits(a.s_q, a.q_off, a.k_off, a.s_kv, a.causal, a.hq, a.hkv, a.d, room).n_split;
}

int attn_fwd_bf16(const AttnArgs& a) {
  const int64_t s_t = kmajor_len(a.s_k);
  int rc = kmajor_launch(a.v, a.workspace, a.s_k, a.hkv, a.d, s_t, a.stream, "attn_fwd_kmajor_v");
  if (rc != USP_OK) return rc;
  const size_t v = vcopy_bytes(a.s_k, a.hkv, a.d);
  const size_t room = a.workspace_bytes > v ? a.workspace_bytes - v : 0;
  const SplitPlan sp =
      plan_splits(a.s_q, a.q_off, a.k_off, a.s_kv, a.causal, a.hq, a.hkv, a.d, room);
  FwdParams p{};
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k);
  p.vt = static_cast<const __bf16*>(a.workspace);
  p.lse = a.lse_out;
  p.m = mask_geom(a);
  p.s_t = s_t;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.scale_log2 = a.scale * kLog2e;
  p.n_split = sp.n_split;
  p.split_tiles = sp.split_tiles;
  float* part = nullptr;
  float* plse = nullptr;
  if (sp.n_split > 1) {
    part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + v);
    plse = reinterpret_cast<float*>(reinterpret_cast<char*>(part) +
                                    align256((size_t)sp.n_split * a.s_q * a.hq * a.d * 4));
    p.o32 = part;
    p.lse = plse;
    p.o_split = a.s_q * a.hq * a.d;
    p.lse_split = a.s_q * a.hq;
  } else {
    p.o = a.out_f32 ? nullptr : static_cast<__bf16*>(a.o_out);
    p.o32 = a.out_f32 ? static_cast<float*>(a.o_out) : nullptr;
  }
  // packed documents, one pass: the query blocks longest first, planned in
  // the room the splits would use
  if (a.cu != nullptr && sp.n_split <= 1 && room >= fwd_order_bytes(a.s_q, a.hq, a.hkv)) {
    const int qrows = qrows_for(a.hq, a.hkv);
    rc = block_order_launch(p.m, kOrderQueryBlocks, (int)((a.s_q + qrows - 1) / qrows), qrows, BN,
                            static_cast<char*>(a.workspace) + v, a.stream, &p.order);
    if (rc != USP_OK) return rc;
  }
  const int g = a.hq / a.hkv;
  rc = a.d == 64 ? fwd_dispatch<64>(p, g, a.hkv, a.stream) : fwd_dispatch<128>(p, g, a.hkv, a.stream);
  if (rc != USP_OK || sp.n_split <= 1) return rc;
  return split_merge_launch(part, plse, p.o_split, p.lse_split, sp.n_split, a.o_out, a.lse_out,
                            a.s_q, a.hq, a.d, a.out_f32, a.stream);
}

}  // namespace usp
