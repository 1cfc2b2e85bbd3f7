// Attention backward, bf16 in / fp32 accumulate, d = 128 or 64, gfx950 matrix cores.
//
// Gradients of one rank's local attention ("feat(dspark): add Ulysses sequence
// parallel training", Accuracy Test: loss and gradient parity with full-sequence
// attention). With the saved natural-log LSE, P_ij = exp(scale q_i.k_j - LSE_i)
// on the allowed keys, dP_ij = dO_i.v_j, D_i = dO_i.O_i, dS = P (dP - D):
//     dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
// with dK and dV summed over the query heads that share a key/value head.
//
// For a query interval against a key interval on global positions (one ring
// step of Ring / USP attention, or a contiguous context-parallel rank's rows;
// see the forward) the same kernels give that pair's contributions: with the
// FINAL O and LSE of the rows, dQ summed over the key intervals and dK, dV
// summed over the query intervals are the full gradients. fp32 outputs may be
// accumulated in place for that sum.
//
// Design (gfx950): two matrix-core kernels, each with one operand stationary
// in registers, so neither needs atomics and both are deterministic.
//   * dK/dV kernel (key-stationary): a workgroup owns 128 keys of one KV head
//     (32 per wave; K and V fragments live in registers) and walks every query
//     tile of every query head of the group that can see them. Scores are
//     computed as S = Q K^T so a lane owns one KEY: P and dS go from the
//     accumulators straight into the B operand of dV^T += dO^T P and
//     dK^T += Q^T dS, whose A operands are read transposed from the Q / dO
//     tiles in LDS.
//   * dQ kernel (query-stationary): like the forward, S^T = K Q^T and
//     dP^T = V dO^T with Q and dO in registers; a lane owns one QUERY, so LSE
//     and D are per-lane scalars, and dS^T feeds dQ^T += K^T dS^T directly.
//   * The cost of skipping atomics is recomputing S and dP in the dQ kernel
//     (7 GEMMs of the 5 the method needs); in exchange there is no fp32
//     accumulation traffic through L2 and the result is reproducible.
//   * Preprocess: D = rowsum(dO * O) and LSE * log2(e).
//   * Tiles go straight from global memory into double-buffered, swizzled LDS
//     slots; masks are applied only on boundary tiles, and the causal
//     triangle is launched heaviest-first (with packed documents, in a
//     longest-first order computed on the device, as in the forward).
//   * Short sequences, where either grid would leave compute units idle and
//     the causal triangle's longest blocks would set the time: the dK/dV
//     kernel splits each key block's rows into chunks, and the dQ kernel
//     splits each query block's keys (planned in splits.hip). Each piece
//     writes an fp32 partial sum into the workspace, and a reduction adds
//     them in a fixed order, so the result still does not depend on
//     scheduling. Pieces with nothing to do write nothing; the reductions
//     find the others from the mask geometry.
#include <algorithm>
#include <type_traits>

#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

// ---------------------------------------------------------------------------
// D_i = sum_d dO[i][h][d] * O[i][h][d]  (fp32 from the bf16 values)
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const __bf16* __restrict__ o,
                                                         const __bf16* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ dd,
                                                         float* __restrict__ lse2, int s_q,
                                                         int hq, int64_t s_t) {
  constexpr int LPR = D / 8;  // lanes per (row, head), 8 elements each
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = t / LPR;
  const int part = (int)(t % LPR);
  float s = 0.f;
  const bool live = rh < (int64_t)s_q * hq;
  if (live) {
    u32x4 a = *reinterpret_cast<const u32x4*>(o + rh * D + part * 8);
    u32x4 b = *reinterpret_cast<const u32x4*>(dout + rh * D + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += bf16_bits_to_f32((unsigned short)(a[e] & 0xffff)) * bf16_bits_to_f32((unsigned short)(b[e] & 0xffff));
      s += bf16_bits_to_f32((unsigned short)(a[e] >> 16)) * bf16_bits_to_f32((unsigned short)(b[e] >> 16));
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (live && part == 0) {
    const int i = (int)(rh / hq), h = (int)(rh % hq);
    dd[(int64_t)h * s_t + i] = s;
    lse2[(int64_t)h * s_t + i] = lse[(int64_t)h * s_q + i] * kLog2e;
  }
}

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;    // [hq][s_q]
  const float* lse2;   // LSE * log2(e), [hq][s_tq]
  const float* dd;     // [hq][s_tq]
  void* dq;            // [s_q][hq][D]
  void* dk;            // [s_k][hkv][D]
  void* dv;            // [s_k][hkv][D]
  MaskGeom m;
  int64_t s_tq;        // row length of lse2 and dd
  int hq, hkv, n_blocks;
  // dK/dV row chunks: grid x = n_kb key blocks x n_ch chunks of cht row tiles;
  // with n_ch > 1 each chunk's fp32 partial dV, dK goes to part
  // ([2][n_ch][s_k][hkv][D], dV first), summed afterwards in chunk order
  int n_kb, n_ch, cht;
  float* part;
  // dQ key splits: grid x = n_blocks query blocks x dq_split; with dq_split > 1
  // split z of a block takes tiles [z, z + 1) * dq_tiles of its key range and
  // writes its scaled fp32 partial dQ to dq_part + z * dq_stride, summed
  // afterwards in split order
  int dq_split, dq_tiles;
  float* dq_part;
  int64_t dq_stride;
  int grad_f32, accum;  // fp32 gradients; add to the existing contents
  float scale, scale_log2;
  // longest-first order of the dK/dV key blocks and of the dQ query blocks
  // (calls with packed documents, one pass each), or NULL: the natural order
  const int* kv_order;
  const int* q_order;
};

// Write DB x 4 accumulator values (registers 4r..4r+3 of block b go to
// elements b*32 + r*8 + [0, 4) past p) scaled by f, as bf16, as fp32, or added
// to fp32.
template <int DB>
__device__ __forceinline__ void store_rows(void* out, int64_t off, const f32x16 (&acc)[DB],
                                           float f, int f32, int accum) {
  if (f32) {
    float* p = static_cast<float*>(out) + off;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v4 = {acc[b][4 * r] * f, acc[b][4 * r + 1] * f, acc[b][4 * r + 2] * f,
                    acc[b][4 * r + 3] * f};
        f32x4* dst = reinterpret_cast<f32x4*>(p + b * 32 + r * 8);
        if (accum) v4 += *dst;
        *dst = v4;
      }
  } else {
    __bf16* p = static_cast<__bf16*>(out) + off;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 v2 = {pack_bf16x2(acc[b][4 * r] * f, acc[b][4 * r + 1] * f),
                    pack_bf16x2(acc[b][4 * r + 2] * f, acc[b][4 * r + 3] * f)};
        *reinterpret_cast<u32x2*>(p + b * 32 + r * 8) = v2;
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV: key-stationary. A workgroup owns KG groups of 32 keys of one KV
// head (KG = 4: 128 keys, 8 waves, one workgroup per CU; KG = 2 runs two
// 4-wave workgroups per CU and measured 10% slower at 120K) and walks every
// query tile (BQ rows) of every query head of the group that can see them.
// Each key group is served by a PAIR of waves:
//   role 0: S = Q K^T -> P -> dV^T += dO^T P   (K fragments stationary)
//   role 1: dP = dO V^T -> dS = P (dP - D) -> dK^T += Q^T dS   (V stationary)
// P crosses from role 0 to role 1 through LDS in accumulator register order
// (16 bytes per lane per 16-row chunk, conflict-free). Splitting the work
// halves each wave's live state (one stationary operand, one accumulator), so
// two waves fit per SIMD and one wave's MFMAs overlap the other's softmax and
// LDS traffic.
//
// Q and dO tiles go from global memory straight into LDS
// (global_load_lds_dwordx4: no staging registers, no LDS stores). That load
// writes each lane's 16 bytes at consecutive LDS addresses, so rows cannot be
// padded; instead chunk c of row r sits in slot c ^ swz_row(r). The
// phase-1 operands (Q, dO with rows = queries) are read as row fragments; the
// phase-2 operands (Q^T, dO^T with rows = d) are read from the same tiles with
// transposed LDS reads, in the row order in which P and dS leave the
// accumulators. Both read patterns are conflict-free under swz16.
template <int D, int BQ, int KG>
__global__ __launch_bounds__(128 * KG, (KG == 2 ? 2 : 1)) void bwd_dkdv_kernel(BwdParams pr) {
  static_assert(KG == 2 || KG == 4, "2 or 4 key groups per workgroup");
  constexpr int KK = D / 16;    // 16-wide reduction steps over d
  constexpr int DB = D / 32;    // 32-row blocks of dK^T / dV^T
  constexpr int KC = D / 8;     // 16-byte chunks per tile row
  constexpr int RPP = 64 / KC;  // tile rows per 1 KiB wave-load
  constexpr int KEYS = 32 * KG;        // keys per workgroup
  static_assert(BQ == 64, "the direct-load tile mapping assumes 64-row tiles");
  constexpr int MB = BQ / 32;          // 32-row blocks per tile
  constexpr int NCH = 2 * MB;          // 16-row chunks per tile
  // Q in slots 0, 1 and dO in slots 2, 3 of one array: the phase-1 and phase-2
  // reads of either tensor are then a fixed register plus a constant
  __shared__ __attribute__((aligned(16))) __bf16 lqo[4][BQ * D];
  __shared__ __attribute__((aligned(16))) float llse[2][BQ];
  __shared__ __attribute__((aligned(16))) float ldd[2][BQ];
  __shared__ __attribute__((aligned(16))) u32x4 lp[KG][NCH][64];
  // These arrays are filled only by direct global->LDS loads, which this
  // compiler does not count as stores to them: without the escape below it
  // treats every read of them as undefined and deletes the dependent work.
  asm volatile("" ::"s"(&lqo[0][0]), "s"(&llse[0][0]), "s"(&ldd[0][0])
               : "memory");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w % KG, role = w / KG;
  const int hl = lane >> 5, ln = lane & 31;
  const int s_q = pr.m.s_q, s_k = pr.m.s_k, s_kv = pr.m.s_kv;
  const int g = pr.hq / pr.hkv;
  const int kvh = blockIdx.y;
  // (key block, row chunk) of this workgroup, chunk-major: the workgroups
  // resident together work on the same rows
  const int cch = (int)blockIdx.x / pr.n_kb;
  const int kbi = pr.kv_order ? order_entry(pr.kv_order, (int)blockIdx.x % pr.n_kb)
                              : (int)blockIdx.x % pr.n_kb;
  const int j0 = kbi * KEYS;
  const int j1 = min(j0 + KEYS, s_k);
  const int wj0 = j0 + grp * 32;
  const int key = wj0 + ln;
  const int kc = min(key, s_k - 1);

  // this lane's key: rows [rlo, rhi) may see it (both ends nondecreasing in
  // the key)
  const RowSpan kr = key_rows(pr.m, kc);
  const bool key_ok = key < s_kv;
  const int rlo = kr.lo, rhi = kr.hi;
  // workgroup row range and mask-free test
  const RowSpan rfirst = key_rows(pr.m, j0), rlast = key_rows(pr.m, j1 - 1);
  const int rstart = max(rfirst.lo, 0);
  const int rend = rlast.hi - 1;
  const int free_lo = rlast.lo, free_hi = rfirst.hi - 1;
  const bool all_keys_valid = j1 - 1 < s_kv;
  // this key group's row range
  const bool wave_live = wj0 < s_k && wj0 < s_kv;
  const int wr_lo = key_rows(pr.m, min(wj0, s_k - 1)).lo;
  const int wr_hi = key_rows(pr.m, min(wj0 + 31, s_k - 1)).hi - 1;

  const int tstart = (rstart / BQ) * BQ;
  // this chunk's row tiles [clo, chi] (tile = BQ rows), chunks counted down
  // from the last tile; with one chunk, every tile of [rstart, rend]
  const int tlast = (s_q - 1) / BQ;
  const int clo = max(tstart / BQ, tlast - (cch + 1) * pr.cht + 1);
  const int chi = min(rend / BQ, tlast - cch * pr.cht);
  const int ntr = (j0 < s_kv && rend >= rstart && chi >= clo) ? chi - clo + 1 : 0;
  const int nt = ntr * g;
  // a chunk with no rows writes no partial (the reduction skips it)
  if (pr.part != nullptr && ntr == 0) return;

  // stationary fragment (B operand, lane = key): K for role 0, V for role 1
  bf16x8 sreg[KK];
  {
    const __bf16* src = role == 0 ? pr.k : pr.v;
    const int64_t off = ((int64_t)kc * pr.hkv + kvh) * D + hl * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sreg[kk] = *reinterpret_cast<const bf16x8*>(src + off + kk * 16);
  }
  // Retire the stationary loads here; otherwise the wait-count pass treats
  // them as possibly in flight inside the loop and makes every MFMA wait for
  // the next tile's loads too.
  __builtin_amdgcn_s_waitcnt(0);
  // The S -> P -> dV waves issue ahead of their dP -> dS -> dK partners when
  // both are ready (wave priority, reset when the wave ends): P is ready
  // sooner and the dV chain keeps the matrix unit busy while the partner does
  // the dS arithmetic.
  if (__builtin_amdgcn_readfirstlane(role) == 0) __builtin_amdgcn_s_setprio(2);
  f32x16 acc[DB];  // dV^T (role 0) or dK^T (role 1): rows = d, cols = keys
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

  // Tile order: query tiles from the END of the sequence downwards, the heads
  // of the group innermost. Every resident workgroup then reads the same
  // (row tile, head) at about the same time, whatever its key block, so the
  // tiles are shared through L2 instead of each workgroup streaming its own
  // row range.
  auto tile_row = [&](int it) { return (chi - it / g) * BQ; };
  // One tile = Q and dO (64 rows x 2d bytes: 64 / RPP wave-loads of 1 KiB,
  // RPP rows each, per tensor) plus the 64 LSE and D values. Rows past the end
  // read the last row: every load is unconditional and such rows are always
  // masked. The next tile is loaded at the top of each tile by the role-1 waves
  // (issuing stalls a wave while the CU's load path drains the burst, and their
  // first phase has the slack): the first half of them bring Q, the second half
  // dO (the parts split evenly), and the first wave of each half also the LSE
  // or D of the tile's rows. Each load is an inline-asm direct load (lds_dma16): a
  // wave-uniform 64-bit base plus a 32-bit lane offset formed per load, waited
  // for once before the barrier that ends the tile.
  const int wu = __builtin_amdgcn_readfirstlane(w);  // LDS destinations go to M0
  const uint32_t row_bytes = (uint32_t)pr.hq * D * 2;
  auto load_tile = [&](int it, int buf) {
    if (wu < KG) return;
    constexpr int HALF = KG / 2, PARTS = BQ / RPP / HALF;  // loading waves per tensor, parts each
    const int r1 = wu - KG;
    const int h = kvh * g + it % g;
    const int r0 = tile_row(it);
    const int p0 = (r1 % HALF) * PARTS;
    const char* base = reinterpret_cast<const char*>(r1 < HALF ? pr.q : pr.dout) + (int64_t)h * (D * 2);
    const uint32_t dst = lds_addr(&lqo[r1 < HALF ? buf : 2 + buf][0]);
    // the lane's byte offset from the first row of a part: row lane / KC,
    // swizzled chunk
    const int q = lane / KC;
    if (r0 + BQ <= s_q) {
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) {
        const int part = p0 + pp;
        const uint32_t off =
            (uint32_t)q * row_bytes + ((uint32_t)((lane % KC) ^ swz_row<D>(RPP * part + q)) << 4);
        lds_dma16(base + (int64_t)(r0 + RPP * part) * row_bytes, off, dst + part * 1024);
      }
    } else {  // the last tile: rows past the end read the last row (always masked)
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) {
        const int part = p0 + pp;
        const int first = min(r0 + RPP * part, s_q - 1);
        const uint32_t rel = (uint32_t)(min(r0 + RPP * part + q, s_q - 1) - first);
        const uint32_t off =
            rel * row_bytes + ((uint32_t)((lane % KC) ^ swz_row<D>(RPP * part + q)) << 4);
        lds_dma16(base + (int64_t)first * row_bytes, off, dst + part * 1024);
      }
    }
    if (r1 % HALF == 0) {
      const int i0 = min(r0, s_q - 1);
      const uint32_t rel = (uint32_t)(min(r0 + lane, s_q - 1) - i0);
      const float* src = (r1 == 0 ? pr.lse2 : pr.dd) + (int64_t)h * pr.s_tq + i0;
      lds_dma4(src, rel * 4, lds_addr(r1 == 0 ? &llse[buf][0] : &ldd[buf][0]));
    }
  };
  // per-lane LDS element offsets of the row-fragment reads and of the
  // transposed reads (column block b, half h) within a tile
  // as LDS byte addresses in slot 0 of the tensor the wave reads (phase 1: Q
  // for role 0, dO for role 1; phase 2 the other), opaque to the compiler so
  // that a slot and block offset is a constant in the read's offset field
  uint32_t ra1[KK], ra2[DB][2];
  {
    const int rolu = __builtin_amdgcn_readfirstlane(role);
    const uint32_t b0 = lds_addr(&lqo[0][0]), dob = 2 * BQ * D * 2;  // dO slot 0
    const uint32_t b1 = b0 + (rolu == 0 ? 0u : dob), b2 = b0 + (rolu == 0 ? dob : 0u);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      ra1[kk] = b1 + 2 * (ln * D + (((hl + 2 * kk) ^ swz_row<D>(ln)) << 3));
      asm volatile("" : "+v"(ra1[kk]));
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ra2[b][h] = b2 + 2 * tr_offset<D>(lane, b, h);
        asm volatile("" : "+v"(ra2[b][h]));
      }
  }

  if (nt > 0) load_tile(0, 0);
  wait_lds_dma();
  __syncthreads();

  // one tile of role R; the loop below is unrolled by two so that the slot is
  // a compile-time constant, and instantiated per role so that each wave runs
  // straight-line code for its own role (with the role as a run-time branch
  // this compiler joined P, dS and the accumulators with register copies)
  // Role 1's dP accumulators live across tiles. Every active tile starts
  // them from zero, and an inactive tile reads nothing, so the results are
  // unchanged. With per-tile accumulators this compiler filled them with
  // zeros ahead of each tile's branch (32 moves per tile).
  f32x16 pa1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) pa1[mb] = f32x16{};
  auto tile = [&](int it, auto parity, auto role_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(parity)::value;  // == it & 1
    constexpr int R = decltype(role_c)::value;    // == role
    const float* tlse = llse[buf];
    const float* tdd = ldd[buf];
    // the next tile into the other slot, whose last reads were in the previous
    // tile; the barrier at the end of this tile waits for it
    if constexpr (R == 1)
      if (it + 1 < nt) load_tile(it + 1, buf ^ 1);
    const int r0 = tile_row(it);
    const bool active = wave_live && r0 + BQ - 1 >= wr_lo && r0 <= wr_hi;

    // phase 1: role 0 -> P (to LDS and registers); role 1 -> dP (registers)
    f32x16 pa0[MB];
    f32x16 (&pa)[MB] = R == 1 ? pa1 : pa0;
    bf16x8 pb[NCH];
    if (active) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // all 8 A fragments of the block are requested before its MFMA chain,
        // so the chain waits for one LDS round trip, not one per MFMA pair
        bf16x8 af[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          af[kk] = lds_read_b128(ra1[kk] + (uint32_t)(buf * BQ * D + mb * 32 * D) * 2);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the chain
        pa[mb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) pa[mb] = mfma32(af[kk], sreg[kk], pa[mb]);
      }
      if constexpr (R == 0) {
        // P = exp2(S*scale*log2e - LSE*log2e); masked entries are 0. Most
        // tiles need no mask, so the mask test is kept off their path.
        const bool full = all_keys_valid && r0 >= free_lo && r0 + BQ - 1 <= free_hi;
        auto probs = [&](auto masked) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int rr = mb * 32 + r4 * 8 + hl * 4;  // first of 4 consecutive rows
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&tlse[rr]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = r4 * 4 + e;
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(pa[mb][i], pr.scale_log2, -l4[e]));
                if constexpr (decltype(masked)::value) {
                  const int row = r0 + rr + e;
                  p = (key_ok && row >= rlo && row < rhi) ? p : 0.f;
                }
                pa[mb][i] = p;
              }
            }
          }
        };
        if (full) probs(std::false_type{});
        else probs(std::true_type{});
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            u32x4 a;
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = pack_bf16x2(pa[mb][8 * c + 2 * t], pa[mb][8 * c + 2 * t + 1]);
            pb[mb * 2 + c] = __builtin_bit_cast(bf16x8, a);
            lp[grp][mb * 2 + c][lane] = a;
          }
        }
      }
    }
    __syncthreads();  // P is visible to role 1

    // phase 2: role 0 -> dV^T += dO^T P; role 1 -> dS, dK^T += Q^T dS
    if (active) {
      if constexpr (R == 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const bf16x8 pv = __builtin_bit_cast(bf16x8, lp[grp][mb * 2 + c][lane]);
            const f32x4 d4a = *reinterpret_cast<const f32x4*>(&tdd[mb * 32 + (2 * c) * 8 + hl * 4]);
            const f32x4 d4b = *reinterpret_cast<const f32x4*>(&tdd[mb * 32 + (2 * c + 1) * 8 + hl * 4]);
            u32x4 o;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i0 = 8 * c + 2 * t, i1 = i0 + 1;  // accumulator registers
              // registers 8c..8c+3 pair with D rows of d4a, 8c+4..8c+7 with d4b
              const float dd0 = t < 2 ? d4a[2 * t] : d4b[2 * t - 4];
              const float dd1 = t < 2 ? d4a[2 * t + 1] : d4b[2 * t - 3];
              const float p0 = (float)pv[2 * t], p1 = (float)pv[2 * t + 1];
              o[t] = pack_bf16x2(p0 * (pa[mb][i0] - dd0), p1 * (pa[mb][i1] - dd1));
            }
            pb[mb * 2 + c] = __builtin_bit_cast(bf16x8, o);
          }
        }
      }
      // dO^T (role 0) or Q^T (role 1): transposed reads of the row tile
      bf16x8 af[DB][NCH];
#pragma unroll
      for (int b2 = 0; b2 < DB; b2 += 2) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch)
            af[b2 + bb][ch] = frag_tr_at(ra2[b2 + bb][0] + (uint32_t)(buf * BQ * D + ch * 16 * D) * 2,
                                         ra2[b2 + bb][1] + (uint32_t)(buf * BQ * D + ch * 16 * D) * 2);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) acc[b2 + bb] = mfma32(af[b2 + bb][ch], pb[ch], acc[b2 + bb]);
      }
      // Order: the first pair's 16 transposed reads, then its chain with two
      // of the second pair's reads after each MFMA, then the second chain.
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      if constexpr (DB == 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    wait_lds_dma();  // the next tile has landed (only the loading waves wait)
    __syncthreads();
  };
  auto run = [&](auto role_c) __attribute__((always_inline)) {
    int it = 0;
    for (; it + 2 <= nt; it += 2) {
      tile(it, std::integral_constant<int, 0>{}, role_c);
      tile(it + 1, std::integral_constant<int, 1>{}, role_c);
    }
    if (it < nt) tile(it, std::integral_constant<int, 0>{}, role_c);
  };
  if (__builtin_amdgcn_readfirstlane(role) == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  if (key < s_k) {
    const int64_t off = ((int64_t)key * pr.hkv + kvh) * D + hl * 4;
    const float f = role == 0 ? 1.f : pr.scale;
    if (pr.part != nullptr) {  // this chunk's partial sum, into its own fp32 slice
      const int64_t slice = (int64_t)s_k * pr.hkv * D;
      store_rows<DB>(pr.part + (int64_t)(role * pr.n_ch + cch) * slice, off, acc, f, 1, 0);
    } else {
      store_rows<DB>(role == 0 ? pr.dv : pr.dk, off, acc, f, pr.grad_f32, pr.accum);
    }
  }
}

// dV and dK from the row chunks' partial sums, added in chunk order (the
// result does not depend on scheduling). Only the chunks holding rows of the
// key's block wrote a partial; which ones is found from the mask geometry
// with the dK/dV kernel's own arithmetic (keys_per_block keys per block,
// tiles of bq rows, cht tiles per chunk counted down from the last tile). One
// thread per 4 values; n4 values of 4 per tensor, key4 of them per key.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part,
                                                          void* dv, void* dk, int64_t n4,
                                                          int n_ch, int f32, int accum,
                                                          MaskGeom m, int keys_per_block, int bq,
                                                          int cht, int key4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const int t = i >= n4 ? 1 : 0;  // 0: dV, 1: dK
  const int64_t e = i - t * n4;
  const int key = (int)(e / key4);
  const int j0 = key / keys_per_block * keys_per_block;
  const int j1 = min(j0 + keys_per_block, m.s_k);
  const RowSpan rfirst = key_rows(m, j0), rlast = key_rows(m, j1 - 1);
  const int rstart = max(rfirst.lo, 0), rend = rlast.hi - 1;
  const int tfirst = rstart / bq, tlast = (m.s_q - 1) / bq;
  const bool rows = j0 < m.s_kv && rend >= rstart;
  const f32x4* src = reinterpret_cast<const f32x4*>(part) + (int64_t)t * n_ch * n4 + e;
  f32x4 acc = {};
  for (int c = 0; c < n_ch; ++c) {
    const int clo = max(tfirst, tlast - (c + 1) * cht + 1);
    const int chi = min(rend / bq, tlast - c * cht);
    if (rows && chi >= clo) acc += src[(int64_t)c * n4];
  }
  void* out = t ? dk : dv;
  if (f32) {
    f32x4* o = reinterpret_cast<f32x4*>(out) + e;
    if (accum) acc += *o;
    *o = acc;
  } else {
    const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    reinterpret_cast<u32x2*>(out)[e] = v;
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary. Workgroup = 4 waves sharing one KV head (HG heads x
// 4/HG blocks of 32 query rows), as in the forward; keys are walked in tiles of
// BN (BN / 32 MFMA key blocks). With BN = 32 two workgroups fit per CU.
//
// K and V tiles go straight from global memory into LDS with the dK/dV
// kernel's row swizzle; K^T for dQ^T += K^T dS^T comes from the K tile by
// transposed reads.
template <int D, int HG, int BN>
__global__ __launch_bounds__(256, (BN == 32 ? 2 : 1)) void bwd_dq_kernel(BwdParams pr) {
  static_assert(BN == 32, "the direct-load tile mapping assumes 32-key tiles");
  constexpr int KK = D / 16;    // 16-wide reduction steps over d
  constexpr int DB = D / 32;    // 32-row blocks of dQ^T
  constexpr int KC = D / 8;     // 16-byte chunks per tile row
  constexpr int RPP = 64 / KC;  // tile rows per 1 KiB wave-load
  constexpr int PPW = BN / RPP / 4;  // wave-loads per wave, tensor and tile
  constexpr int QROWS = 32 * (4 / HG);
  constexpr int KB = BN / 32;
  // K slots 0, 1 and V slots 0, 1 in one array, so that every slot sits at a
  // fixed offset from the first (the fragment reads below add it as a
  // constant); the direct loads are inline asm, which the wait-count pass does
  // not see, so sharing an array costs no waits
  __shared__ __attribute__((aligned(16))) __bf16 lkv[4][BN * D];
  // filled only by direct loads, which this compiler does not count as stores
  asm volatile("" ::"s"(&lkv[0][0]) : "memory");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, ln = lane & 31;
  const int s_q = pr.m.s_q, s_k = pr.m.s_k;
  const int g = pr.hq / pr.hkv;
  const int chunks = g / HG;
  const int kvh = blockIdx.y / chunks, hc = blockIdx.y % chunks;
  const int head = kvh * g + hc * HG + (w % HG);
  // heaviest query block first; its key splits follow one another, the
  // order rotated by the block when their count is even (see the forward)
  const int bi = (int)blockIdx.x / pr.dq_split;
  const int qb = pr.q_order ? order_entry(pr.q_order, bi) : pr.n_blocks - 1 - bi;
  const int zk = (int)blockIdx.x % pr.dq_split;
  const int zs = (pr.dq_split & 1) ? zk : (zk + qb) % pr.dq_split;
  const int q0 = qb * QROWS;
  const int q1 = min(q0 + QROWS, s_q);
  const int wq0 = q0 + (w / HG) * 32;
  const int qi = wq0 + ln;
  const bool row_ok = qi < s_q;
  const int qc = row_ok ? qi : s_q - 1;

  const KeyRange kr = row_keys(pr.m, qc);
  const int lo = kr.lo, hi = kr.hi;
  const KeyRange kfirst = row_keys(pr.m, q0), klast = row_keys(pr.m, q1 - 1);
  // workgroup key range; with key splits, the part of it in this split's
  // tiles (counted from the tile holding the first key)
  const int t_split = (kfirst.lo / BN + zs * pr.dq_tiles) * BN;
  const int kmin = pr.dq_split > 1 ? max(kfirst.lo, t_split) : kfirst.lo;
  const int kmax = pr.dq_split > 1 ? min(klast.hi, t_split + pr.dq_tiles * BN - 1) : klast.hi;
  const int free_lo = klast.lo, free_hi = kfirst.hi;
  const int tstart = (kmin / BN) * BN;
  const int nt = kmax >= kmin ? (kmax - tstart) / BN + 1 : 0;
  if (pr.dq_split > 1 && nt == 0) return;  // no keys here: the sum skips this split
  const int wkmin = row_keys(pr.m, min(wq0, s_q - 1)).lo;
  const int wkmax = row_keys(pr.m, min(wq0 + 31, s_q - 1)).hi;

  bf16x8 qreg[KK], doreg[KK];
  {
    const int64_t off = ((int64_t)qc * pr.hq + head) * D + hl * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qreg[kk] = *reinterpret_cast<const bf16x8*>(pr.q + off + kk * 16);
      doreg[kk] = *reinterpret_cast<const bf16x8*>(pr.dout + off + kk * 16);
    }
  }
  const float lse2 = pr.lse[(int64_t)head * s_q + qc] * kLog2e;
  const float drow = pr.dd[(int64_t)head * pr.s_tq + qc];
  // retire the stationary loads before the loop (see the dK/dV kernel)
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 dqa[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) dqa[b] = f32x16{};

  // A part is one 1 KiB wave-load (RPP keys of K or V); wave w brings K and V
  // parts PPW w .. +PPW-1 as inline-asm direct loads (see lds_dma16): a
  // wave-uniform base plus a 32-bit lane offset.
  const int wu = __builtin_amdgcn_readfirstlane(w);  // LDS destinations go to M0
  const uint32_t key_bytes = (uint32_t)pr.hkv * D * 2;
  const int q_in_part = lane / KC;  // key within a part; lane % KC is the LDS slot
  // lane offsets of the parts of a tile that lies inside the sequence (a
  // constant per lane: key q_in_part of the part, swizzled chunk)
  uint32_t kvoff[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j)
    kvoff[j] = (uint32_t)q_in_part * key_bytes +
               ((uint32_t)((lane % KC) ^ swz_row<D>(RPP * (PPW * wu + j) + q_in_part)) << 4);
  auto load_tile = [&](int t0, int buf) {
    const uint32_t dk = lds_addr(&lkv[buf][0]);
    const uint32_t dv = lds_addr(&lkv[2 + buf][0]);
    const char* kb = reinterpret_cast<const char*>(pr.k) + (int64_t)kvh * (D * 2);
    const char* vb = reinterpret_cast<const char*>(pr.v) + (int64_t)kvh * (D * 2);
    if (t0 + BN <= s_k) {
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int part = PPW * wu + j;
        const int64_t row = (int64_t)(t0 + RPP * part) * key_bytes;
        lds_dma16(kb + row, kvoff[j], dk + part * 1024);
        lds_dma16(vb + row, kvoff[j], dv + part * 1024);
      }
      return;
    }
    const int q = q_in_part;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int part = PPW * wu + j;
      // keys past the end read the last key (always masked)
      const int first = min(t0 + RPP * part, s_k - 1);
      const uint32_t rel = (uint32_t)(min(t0 + RPP * part + q, s_k - 1) - first);
      const uint32_t off =
          rel * key_bytes + ((uint32_t)((lane % KC) ^ swz_row<D>(RPP * part + q)) << 4);
      lds_dma16(kb + (int64_t)first * key_bytes, off, dk + part * 1024);
      lds_dma16(vb + (int64_t)first * key_bytes, off, dv + part * 1024);
    }
  };
  // fragment read offsets (elements) within a tile
  // LDS byte addresses of the lane's row-fragment and transposed reads in
  // the first K slot, opaque to the compiler: every read of a slot or block
  // is then one of these registers plus a constant offset (with element
  // offsets the compiler formed each address anew, or kept one per slot)
  uint32_t kra[KK], tra[DB][2];
  {
    const uint32_t b0 = lds_addr(&lkv[0][0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kra[kk] = b0 + 2 * (ln * D + (((hl + 2 * kk) ^ swz_row<D>(ln)) << 3));
      asm volatile("" : "+v"(kra[kk]));
    }
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tra[b][h] = b0 + 2 * tr_offset<D>(lane, b, h);
        asm volatile("" : "+v"(tra[b][h]));
      }
  }

  if (nt > 0) load_tile(tstart, 0);
  wait_lds_dma();
  __syncthreads();

  auto step = [&](int it, auto parity) {
    constexpr int buf = decltype(parity)::value;
    const int t0 = tstart + it * BN;
    // the next tile into the other slot (last read in the previous tile); the
    // barrier at the end of this tile waits for it
    if (it + 1 < nt) load_tile(t0 + BN, buf ^ 1);

    if (t0 <= wkmax && t0 + BN - 1 >= wkmin) {
      f32x16 sa[KB], pa[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // the A fragments of each chain are requested before the chain runs
        const uint32_t ko = (uint32_t)(buf * BN * D + kb * 32 * D) * 2;        // K slot
        const uint32_t vo = (uint32_t)((2 + buf) * BN * D + kb * 32 * D) * 2;  // V slot
        bf16x8 afk[KK], afv[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) afk[kk] = lds_read_b128(kra[kk] + ko);
        sa[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sa[kb] = mfma32(afk[kk], qreg[kk], sa[kb]);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) afv[kk] = lds_read_b128(kra[kk] + vo);
        pa[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) pa[kb] = mfma32(afv[kk], doreg[kk], pa[kb]);
        // Order: the K fragments, then the S chain with one V fragment read
        // after each of its MFMAs (the V reads overlap the chain instead of
        // starting after it), then the dP chain.
        __builtin_amdgcn_sched_group_barrier(0x100, KK, 0);  // LDS reads (K)
#pragma unroll
        for (int i = 0; i < KK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA (S)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read (V)
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KK, 0);  // the dP chain
      }
      const bool full = t0 >= free_lo && t0 + BN - 1 <= free_hi;
      // K^T fragments for dQ^T += K^T dS^T, requested before the softmax so
      // that its vector work covers their latency
      bf16x8 kft[DB][2 * KB];
      {
        constexpr uint32_t ko = (uint32_t)(buf * BN * D) * 2;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int ch = 0; ch < 2 * KB; ++ch)
            kft[b][ch] = frag_tr_at(tra[b][0] + ko + ch * 16 * D * 2, tra[b][1] + ko + ch * 16 * D * 2);
      }
      // dS^T = P^T (dP^T - D); most tiles need no mask, so the mask test is
      // kept off their path
      auto dsoft = [&](auto masked) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[kb][i], pr.scale_log2, -lse2));
            if constexpr (decltype(masked)::value) {
              const int key = t0 + kb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
              p = (key >= lo && key <= hi) ? p : 0.f;
            }
            pa[kb][i] = p * (pa[kb][i] - drow);
          }
        }
      };
      if (full) dsoft(std::false_type{});
      else dsoft(std::true_type{});
      bf16x8 dst[2 * KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 b;
#pragma unroll
          for (int t = 0; t < 4; ++t) b[t] = pack_bf16x2(pa[kb][8 * c + 2 * t], pa[kb][8 * c + 2 * t + 1]);
          dst[kb * 2 + c] = __builtin_bit_cast(bf16x8, b);
        }
      }
      // dQ^T += K^T dS^T (rows = d, cols = queries)
#pragma unroll
      for (int ch = 0; ch < 2 * KB; ++ch)
#pragma unroll
        for (int b = 0; b < DB; ++b) dqa[b] = mfma32(kft[b][ch], dst[ch], dqa[b]);
    }
    wait_lds_dma();  // the next tile has landed
    __syncthreads();
  };
  for (int it = 0; it < nt; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nt) step(it + 1, std::integral_constant<int, 1>{});
  }

  if (row_ok) {
    const bool split = pr.dq_split > 1;
    store_rows<DB>(split ? static_cast<void*>(pr.dq_part + zs * pr.dq_stride) : pr.dq,
                   ((int64_t)qi * pr.hq + head) * D + hl * 4, dqa, pr.scale,
                   split ? 1 : pr.grad_f32, split ? 0 : pr.accum);
  }
}

// dQ from the key splits' partial sums, added in split order (the result does
// not depend on scheduling). Split z of a query block holds keys only when the
// block has more than z * tiles_per_split key tiles, found from the mask
// geometry exactly as the dQ kernel finds them; the other splits wrote nothing
// and are not read (a block with no keys gets dQ = 0). One thread per 4
// values; a row has row4 groups of 4 values.
__global__ __launch_bounds__(256) void dq_reduce_kernel(const float* __restrict__ part,
                                                        int64_t stride, int nz,
                                                        int tiles_per_split, int key_tile,
                                                        MaskGeom m, int qrows, uint32_t row4,
                                                        void* dq, uint32_t n4, int f32, int accum) {
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int row = (int)(i / row4);
  const int q0 = row / qrows * qrows;
  const int q1 = min(q0 + qrows, m.s_q);
  const KeyRange kf = row_keys(m, q0), kl = row_keys(m, q1 - 1);
  const int tstart = kf.lo / key_tile * key_tile;
  const int nt = kl.hi >= kf.lo ? (kl.hi - tstart) / key_tile + 1 : 0;
  const int nzr = min(nz, (nt + tiles_per_split - 1) / tiles_per_split);
  const f32x4* src = reinterpret_cast<const f32x4*>(part) + i;
  f32x4 acc = {};
  for (int z = 0; z < nzr; ++z) acc += src[z * (stride / 4)];
  if (f32) {
    f32x4* o = reinterpret_cast<f32x4*>(dq) + i;
    if (accum) acc += *o;
    *o = acc;
  } else {
    const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    reinterpret_cast<u32x2*>(dq)[i] = v;
  }
}

constexpr int kDqKeys = 32;      // keys per dQ tile
constexpr int kDkdvRows = 64;    // query rows per dK/dV tile
constexpr int kDkdvGroups = 4;   // 32-key groups (wave pairs) per dK/dV workgroup

// Row chunks per key block in the dK/dV kernel. When the key blocks alone give
// too few workgroups, most compute units would sit idle, and under a causal
// mask the first blocks walk many times the rows of the last, so each key
// block's rows are split into chunks whose fp32 partials a reduction adds. The
// counts come from a sweep of 1..32 chunks (dK/dV kernel plus reduction,
// d = 128): on one KV head the best counts give about 4096 (key block, chunk)
// items, at most 16 chunks (4K: 84 us at 16 chunks, 72 at 8; 8K: 201 at 16;
// 16K: 603 at 16; 32K: 2137 at 16, 2266 at 8), and from 512 blocks one pass
// (120K: 2 chunks tie with 1). With several KV heads the partials' traffic
// grows with the head count and 2 chunks are best below 1024 items (4100
// tokens, 16 Q / 4 KV: 231 us against 286 at 16; 8K, 32 Q / 8 KV: 1287
// against 1663 in one pass). A dispatch simulation of the kind that plans the
// key splits ranked these counts poorly (it picked 6 at 8K and 2 at 32K).
int dkdv_row_chunks(int64_t s_q, int64_t s_k, int hkv) {
  constexpr int keys = 32 * kDkdvGroups;
  const int64_t items = (s_k + keys - 1) / keys * hkv;
  const int64_t tiles = (s_q + kDkdvRows - 1) / kDkdvRows;
  int64_t n;
  if (hkv == 1) {
    if (items >= 512) return 1;
    n = (4096 + items - 1) / items;
    n = n < 16 ? n : 16;
  } else {
    if (items >= 1024) return 1;
    n = 2;
  }
  n = n < tiles ? n : tiles;
  return n > 1 ? (int)n : 1;
}

int hg_for(int g) { return g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1; }
int dq_qrows(int hq, int hkv) { return 32 * (4 / hg_for(hq / hkv)); }

// dQ key splits pay off only while the unsplit grid is short of a few rounds
// of workgroups on the 512 resident slots (two 4-wave workgroups per compute
// unit).
constexpr int kDqSlots = 512;
constexpr int kDqMaxSplits = 8;
int dq_split_cap(int64_t s_q, int hq, int hkv) {
  const int g = hq / hkv;
  const int64_t wgs = (s_q + dq_qrows(hq, hkv) - 1) / dq_qrows(hq, hkv) * hkv * (g / hg_for(g));
  if (wgs >= 2 * kDqSlots) return 1;
  return (int)std::min<int64_t>(kDqMaxSplits, (4 * kDqSlots + wgs - 1) / wgs);
}

size_t dq_split_bytes(int z, int64_t s_q, int hq, int d) {
  return z > 1 ? (size_t)z * s_q * hq * d * 4 : 0;
}

// The dQ key splits of a call with `room` workspace bytes for the partials.
// One 32-key tile of a 4-wave workgroup takes about 1.3 us at d = 128 with two
// workgroups per compute unit; at 5 TB/s that is d x 52 KB of traffic.
SplitPlan plan_dq(int64_t s_q, int64_t q_off, int64_t k_off, int64_t s_kv, int causal, int hq,
                  int hkv, int d, size_t room) {
  int cap = dq_split_cap(s_q, hq, hkv);
  while (cap > 1 && dq_split_bytes(cap, s_q, hq, d) > room) --cap;
  SplitProblem sp{};
  sp.s_q = s_q;
  sp.q_off = q_off;
  sp.k_off = k_off;
  sp.s_kv = s_kv;
  sp.causal = causal;
  sp.qrows = dq_qrows(hq, hkv);
  sp.heads = hkv * (hq / hkv / hg_for(hq / hkv));
  sp.key_tile = kDqKeys;
  sp.slots = kDqSlots;
  sp.cap = cap;
  sp.min_tiles = 16;
  // each (block, split) partial is written and read back; dQ written once
  sp.item_bytes = (double)sp.qrows * hg_for(hq / hkv) * d * 8;
  sp.fixed_bytes = (double)s_q * hq * d * 2;
  sp.tile_bytes = 52.0e3 * d;
  return plan_key_splits(sp);
}

template <int D, int HG>
int launch_dq(const BwdParams& p, int g, const AttnArgs& a) {
  constexpr int QROWS = 32 * (4 / HG);
  BwdParams pr = p;
  pr.n_blocks = (p.m.s_q + QROWS - 1) / QROWS;
  dim3 grid((unsigned)(pr.n_blocks * pr.dq_split), (unsigned)(p.hkv * (g / HG)));
  {
    TraceScope ts("attn_bwd_dq_bf16", a.stream);
    hipLaunchKernelGGL((bwd_dq_kernel<D, HG, kDqKeys>), grid, dim3(256), 0, a.stream, pr);
    if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
  }
  if (pr.dq_split <= 1) return USP_OK;
  const uint32_t n4 = (uint32_t)(a.s_q * a.hq * D / 4);
  TraceScope ts("attn_bwd_dq_reduce", a.stream);
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((n4 + 255) / 256), dim3(256), 0, a.stream,
                     static_cast<const float*>(pr.dq_part), pr.dq_stride, pr.dq_split, pr.dq_tiles,
                     kDqKeys, pr.m, QROWS, (uint32_t)(a.hq * D / 4), a.dq, n4, a.out_f32,
                     a.accumulate);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

// D and LSE * log2(e), then dK/dV, then dQ, for head dim D
template <int D>
int bwd_launch(const BwdParams& p, const AttnArgs& a, float* dd, float* lse2, float* part) {
  {
    const int64_t n = a.s_q * a.hq * (D / 8);
    TraceScope ts("attn_bwd_rowdot_bf16", a.stream);
    hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       a.stream, static_cast<const __bf16*>(a.o),
                       static_cast<const __bf16*>(a.dout), a.lse, dd, lse2, (int)a.s_q, a.hq,
                       p.s_tq);
    if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
  }
  {
    constexpr int keys = 32 * kDkdvGroups;
    BwdParams pk = p;
    pk.n_kb = (int)((a.s_k + keys - 1) / keys);
    pk.n_ch = dkdv_row_chunks(a.s_q, a.s_k, a.hkv);
    const int tiles = (int)((a.s_q + kDkdvRows - 1) / kDkdvRows);
    pk.cht = (tiles + pk.n_ch - 1) / pk.n_ch;
    pk.part = pk.n_ch > 1 ? part : nullptr;
    dim3 grid((unsigned)(pk.n_kb * pk.n_ch), (unsigned)a.hkv);
    {
      TraceScope ts("attn_bwd_dkdv_bf16", a.stream);
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, kDkdvRows, kDkdvGroups>), grid,
                         dim3(128 * kDkdvGroups), 0, a.stream, pk);
      if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
    }
    if (pk.n_ch > 1) {
      const int64_t n4 = a.s_k * a.hkv * D / 4;
      TraceScope ts("attn_bwd_dkdv_reduce", a.stream);
      hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0,
                         a.stream, static_cast<const float*>(part), a.dv, a.dk, n4, pk.n_ch,
                         a.out_f32, a.accumulate, pk.m, keys, kDkdvRows, pk.cht,
                         (int)(a.hkv * D / 4));
      if (hipGetLastError() != hipSuccess) return USP_ERR_HIP;
    }
  }
  const int g = a.hq / a.hkv;
  if (g % 4 == 0) return launch_dq<D, 4>(p, g, a);
  if (g % 2 == 0) return launch_dq<D, 2>(p, g, a);
  return launch_dq<D, 1>(p, g, a);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Required part of the workspace: D and LSE*log2(e) per query row and head,
// then the dK/dV row-chunk partials (256-byte aligned).
size_t bwd_required(int64_t s_q, int64_t s_k, int hq, int hkv, int d) {
  const size_t rows = align256((size_t)hq * (size_t)kmajor_len(s_q) * 4) * 2;
  const int n_ch = dkdv_row_chunks(s_q, s_k, hkv);
  return rows + align256(n_ch > 1 ? (size_t)2 * n_ch * (size_t)s_k * hkv * d * 4 : 0);
}

// Bytes of the two block orders: key blocks of the dK/dV kernel, then query
// blocks of the dQ kernel.
size_t bwd_order_bytes(int64_t s_q, int64_t s_k, int hq, int hkv) {
  constexpr int keys = 32 * kDkdvGroups;
  return block_order_bytes((s_k + keys - 1) / keys) +
         block_order_bytes((s_q + dq_qrows(hq, hkv) - 1) / dq_qrows(hq, hkv));
}

SplitPlan plan_dq_for(const AttnArgs& a) {
  const size_t req = bwd_required(a.s_q, a.s_k, a.hq, a.hkv, a.d);
  const size_t room = a.workspace_bytes > req ? a.workspace_bytes - req : 0;
  return plan_dq(a.s_q, a.q_off, a.k_off, a.s_kv, a.causal, a.hq, a.hkv, a.d, room);
}

}  // namespace

// The required part, then room for the dQ key splits of s_q rows, or for the
// block orders of the dK/dV key blocks and the dQ query blocks (used only
// without splits or row chunks).
size_t attn_bwd_bf16_workspace(int64_t s_q, int64_t s_k, int hq, int hkv, int d) {
  return bwd_required(s_q, s_k, hq, hkv, d) +
         std::max(dq_split_bytes(dq_split_cap(s_q, hq, hkv), s_q, hq, d),
                  bwd_order_bytes(s_q, s_k, hq, hkv));
}

size_t attn_bwd_bf16_min_workspace(int64_t s_q, int64_t s_k, int hq, int hkv, int d) {
  return bwd_required(s_q, s_k, hq, hkv, d);
}

int attn_bwd_bf16_dq_splits(const AttnArgs& a) { return plan_dq_for(a).n_split; }

int attn_bwd_bf16(const AttnArgs& a) {
  const int64_t s_tq = kmajor_len(a.s_q);
  char* ws = static_cast<char*>(a.workspace);
  float* dd = reinterpret_cast<float*>(ws);
  float* lse2 = reinterpret_cast<float*>(ws + align256((size_t)a.hq * s_tq * 4));
  float* part = reinterpret_cast<float*>(ws + 2 * align256((size_t)a.hq * s_tq * 4));
  BwdParams p{};
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k);
  p.v = static_cast<const __bf16*>(a.v);
  p.dout = static_cast<const __bf16*>(a.dout);
  p.lse = a.lse;
  p.lse2 = lse2;
  p.dd = dd;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.m = mask_geom(a);
  p.s_tq = s_tq;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.grad_f32 = a.out_f32;
  p.accum = a.accumulate;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const SplitPlan dp = plan_dq_for(a);
  const size_t req = bwd_required(a.s_q, a.s_k, a.hq, a.hkv, a.d);
  p.dq_split = dp.n_split;
  p.dq_tiles = dp.split_tiles;
  p.dq_part = reinterpret_cast<float*>(ws + req);
  p.dq_stride = a.s_q * a.hq * a.d;
  // packed documents, one pass in both kernels: their blocks longest first,
  // planned in the room the dQ splits would use
  const size_t room = a.workspace_bytes > req ? a.workspace_bytes - req : 0;
  if (a.cu != nullptr && dp.n_split <= 1 && dkdv_row_chunks(a.s_q, a.s_k, a.hkv) == 1 &&
      room >= bwd_order_bytes(a.s_q, a.s_k, a.hq, a.hkv)) {
    constexpr int keys = 32 * kDkdvGroups;
    const int n_kb = (int)((a.s_k + keys - 1) / keys);
    const int qrows = dq_qrows(a.hq, a.hkv);
    int rc = block_order_launch(p.m, kOrderKeyBlocks, n_kb, keys, kDkdvRows, ws + req, a.stream,
                                &p.kv_order);
    if (rc != USP_OK) return rc;
    rc = block_order_launch(p.m, kOrderQueryBlocks, (int)((a.s_q + qrows - 1) / qrows), qrows,
                            kDqKeys, ws + req + block_order_bytes(n_kb), a.stream, &p.q_order);
    if (rc != USP_OK) return rc;
  }
  return a.d == 64 ? bwd_launch<64>(p, a, dd, lse2, part) : bwd_launch<128>(p, a, dd, lse2, part);
}

}  // namespace usp
