// fp32 attention forward and backward (plain SIMT, no matrix cores).
//
// This path serves fp32 problems (the small fp32 check workload: 512 tokens,
// 4 query / 2 key-value heads per rank, d = 64). One lane owns one query row
// (forward, dQ) or one key row (dK/dV); key/value or query/dO tiles are staged
// in LDS and every lane walks them. It is written for exactness, not speed.
//
// Mask (as in the bf16 path): key j is allowed for query row i iff
// j < s_valid, doc(j) == doc(i) and, when causal, j <= i (local attention
// after the Ulysses all-to-all, "feat(dspark): add Ulysses sequence parallel
// training", Modifications; packed documents, "GLM-5.2 131k context
// parallelism", Purpose). Like the bf16 path it also takes a query interval
// against a key interval on global positions (see the bf16 forward), with
// in-place accumulation of the gradients for that case.
#include "usp_common.h"
#include "usp_internal.h"

namespace usp {

namespace {

constexpr int kRows = 64;   // rows per block (one wave)
constexpr int kTile = 32;   // staged rows per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        float* __restrict__ o,
                                                        float* __restrict__ lse, MaskGeom mg,
                                                        int hq, int hkv, float scale) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int s_q = mg.s_q, s_k = mg.s_k;
  const int h = blockIdx.y, kvh = h / (hq / hkv);
  const int q0 = blockIdx.x * kRows;
  const int q1 = min(q0 + kRows, s_q);
  const int i = q0 + threadIdx.x;
  const bool row_ok = i < s_q;
  const int ii = row_ok ? i : q1 - 1;
  const KeyRange rr = row_keys(mg, ii);
  const int kmin = row_keys(mg, q0).lo;
  const int kmax = row_keys(mg, q1 - 1).hi;

  float qr[D], acc[D];
  for (int c = 0; c < D; ++c) {
    qr[c] = q[((int64_t)ii * hq + h) * D + c] * (scale * kLog2e);
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t0 = kmin; t0 <= kmax; t0 += kTile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * D; e += kRows) {
      const int r = e / D, c = e % D, j = t0 + r;
      const bool in = j < s_k;
      ks[r][c] = in ? k[((int64_t)j * hkv + kvh) * D + c] : 0.f;
      vs[r][c] = in ? v[((int64_t)j * hkv + kvh) * D + c] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      const int j = t0 + r;
      if (j < rr.lo || j > rr.hi) continue;
      float s = 0.f;
      for (int c = 0; c < D; ++c) s += qr[c] * ks[r][c];
      if (s > m) {
        const float alpha = exp2f(m - s);
        for (int c = 0; c < D; ++c) acc[c] *= alpha;
        l *= alpha;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
      for (int c = 0; c < D; ++c) acc[c] += p * vs[r][c];
    }
  }
  if (row_ok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int c = 0; c < D; ++c) o[((int64_t)i * hq + h) * D + c] = acc[c] * inv;
    lse[(int64_t)h * s_q + i] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

// D_i = dO_i . O_i per (head, row).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float* __restrict__ o,
                                                          const float* __restrict__ dout,
                                                          float* __restrict__ dd, int s_q,
                                                          int hq) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)s_q * hq) return;
  const int i = (int)(t / hq), h = (int)(t % hq);
  float s = 0.f;
  for (int c = 0; c < D; ++c) s += o[t * D + c] * dout[t * D + c];
  dd[(int64_t)h * s_q + i] = s;
}

template <int D>
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dout, const float* __restrict__ dd,
    float* __restrict__ dq, MaskGeom mg, int hq, int hkv, float scale, int accum) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int s_q = mg.s_q, s_k = mg.s_k;
  const int h = blockIdx.y, kvh = h / (hq / hkv);
  const int q0 = blockIdx.x * kRows;
  const int q1 = min(q0 + kRows, s_q);
  const int i = q0 + threadIdx.x;
  const bool row_ok = i < s_q;
  const int ii = row_ok ? i : q1 - 1;
  const KeyRange rr = row_keys(mg, ii);
  const int kmin = row_keys(mg, q0).lo, kmax = row_keys(mg, q1 - 1).hi;

  float qr[D], dor[D], acc[D];
  for (int c = 0; c < D; ++c) {
    qr[c] = q[((int64_t)ii * hq + h) * D + c];
    dor[c] = dout[((int64_t)ii * hq + h) * D + c];
    acc[c] = 0.f;
  }
  const float lrow = lse[(int64_t)h * s_q + ii];
  const float drow = dd[(int64_t)h * s_q + ii];
  for (int t0 = kmin; t0 <= kmax; t0 += kTile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * D; e += kRows) {
      const int r = e / D, c = e % D, j = t0 + r;
      const bool in = j < s_k;
      ks[r][c] = in ? k[((int64_t)j * hkv + kvh) * D + c] : 0.f;
      vs[r][c] = in ? v[((int64_t)j * hkv + kvh) * D + c] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      const int j = t0 + r;
      if (j < rr.lo || j > rr.hi) continue;
      float s = 0.f, dp = 0.f;
      for (int c = 0; c < D; ++c) {
        s += qr[c] * ks[r][c];
        dp += dor[c] * vs[r][c];
      }
      const float p = expf(s * scale - lrow);
      const float ds = p * (dp - drow);
      for (int c = 0; c < D; ++c) acc[c] += ds * ks[r][c];
    }
  }
  if (row_ok)
    for (int c = 0; c < D; ++c) {
      float* p = dq + ((int64_t)i * hq + h) * D + c;
      *p = acc[c] * scale + (accum ? *p : 0.f);
    }
}

template <int D>
__global__ __launch_bounds__(kRows) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dout, const float* __restrict__ dd,
    float* __restrict__ dk, float* __restrict__ dv, MaskGeom mg, int hq, int hkv, float scale,
    int accum) {
  __shared__ float qs[kTile][D];
  __shared__ float dos[kTile][D];
  __shared__ float ls[kTile], ds_[kTile];
  const int s_q = mg.s_q, s_k = mg.s_k;
  const int kvh = blockIdx.y, g = hq / hkv;
  const int j0 = blockIdx.x * kRows;
  const int j1 = min(j0 + kRows, s_k);
  const int j = j0 + threadIdx.x;
  const bool key_ok = j < s_k;
  const int jj = key_ok ? j : j1 - 1;
  const RowSpan jr = key_rows(mg, jj);  // rows [jr.lo, jr.hi) may see key jj
  const bool valid_key = jj < mg.s_kv;
  // rows that can see any key of this block
  const int rmin = max(key_rows(mg, j0).lo, 0);
  const int rmax = key_rows(mg, j1 - 1).hi - 1;

  float kr[D], vr[D], dka[D], dva[D];
  for (int c = 0; c < D; ++c) {
    kr[c] = k[((int64_t)jj * hkv + kvh) * D + c];
    vr[c] = v[((int64_t)jj * hkv + kvh) * D + c];
    dka[c] = 0.f;
    dva[c] = 0.f;
  }
  for (int hh = 0; hh < g; ++hh) {
    const int h = kvh * g + hh;
    for (int t0 = rmin; t0 <= rmax; t0 += kTile) {
      __syncthreads();
      for (int e = threadIdx.x; e < kTile * D; e += kRows) {
        const int r = e / D, c = e % D, i = t0 + r;
        const bool in = i < s_q;
        qs[r][c] = in ? q[((int64_t)i * hq + h) * D + c] : 0.f;
        dos[r][c] = in ? dout[((int64_t)i * hq + h) * D + c] : 0.f;
      }
      if (threadIdx.x < kTile) {
        const int i = t0 + threadIdx.x;
        ls[threadIdx.x] = i < s_q ? lse[(int64_t)h * s_q + i] : 0.f;
        ds_[threadIdx.x] = i < s_q ? dd[(int64_t)h * s_q + i] : 0.f;
      }
      __syncthreads();
      if (!valid_key) continue;
      for (int r = 0; r < kTile; ++r) {
        const int i = t0 + r;
        if (i < jr.lo || i >= jr.hi) continue;
        float s = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
          s += qs[r][c] * kr[c];
          dp += dos[r][c] * vr[c];
        }
        const float p = expf(s * scale - ls[r]);
        const float dsv = p * (dp - ds_[r]);
        for (int c = 0; c < D; ++c) {
          dva[c] += p * dos[r][c];
          dka[c] += dsv * qs[r][c];
        }
      }
    }
  }
  if (key_ok) {
    for (int c = 0; c < D; ++c) {
      float* pk = dk + ((int64_t)j * hkv + kvh) * D + c;
      float* pv = dv + ((int64_t)j * hkv + kvh) * D + c;
      *pk = dka[c] * scale + (accum ? *pk : 0.f);
      *pv = dva[c] + (accum ? *pv : 0.f);
    }
  }
}

template <int D>
int fwd_f32_launch(const AttnArgs& a) {
  dim3 grid((unsigned)((a.s_q + kRows - 1) / kRows), (unsigned)a.hq);
  TraceScope ts("attn_fwd_f32", a.stream);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(kRows), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o_out,
                     a.lse_out, mask_geom(a), a.hq, a.hkv, a.scale);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

template <int D>
int bwd_f32_launch(const AttnArgs& a) {
  float* dd = static_cast<float*>(a.workspace);
  const int64_t n = a.s_q * a.hq;
  const MaskGeom mg = mask_geom(a);
  {
    TraceScope ts("attn_bwd_rowdot_f32", a.stream);
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       a.stream, (const float*)a.o, (const float*)a.dout, dd, (int)a.s_q, a.hq);
  }
  dim3 gq((unsigned)((a.s_q + kRows - 1) / kRows), (unsigned)a.hq);
  {
    TraceScope ts("attn_bwd_dq_f32", a.stream);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), gq, dim3(kRows), 0, a.stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, a.lse, (const float*)a.dout, dd,
                       (float*)a.dq, mg, a.hq, a.hkv, a.scale, a.accumulate);
  }
  dim3 gk((unsigned)((a.s_k + kRows - 1) / kRows), (unsigned)a.hkv);
  TraceScope ts("attn_bwd_dkdv_f32", a.stream);
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), gk, dim3(kRows), 0, a.stream, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, a.lse, (const float*)a.dout, dd,
                     (float*)a.dk, (float*)a.dv, mg, a.hq, a.hkv, a.scale, a.accumulate);
  return hipGetLastError() == hipSuccess ? USP_OK : USP_ERR_HIP;
}

}  // namespace

size_t attn_bwd_f32_workspace(int64_t s_q, int hq, int, int) {
  return (size_t)s_q * hq * sizeof(float);
}

int attn_fwd_f32(const AttnArgs& a) {
  return a.d == 64 ? fwd_f32_launch<64>(a) : fwd_f32_launch<128>(a);
}

int attn_bwd_f32(const AttnArgs& a) {
  return a.d == 64 ? bwd_f32_launch<64>(a) : bwd_f32_launch<128>(a);
}

}  // namespace usp
