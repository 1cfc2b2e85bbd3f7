// C ABI entry points of libusp: host-side argument checks, then kernel
// dispatch. Every check runs before the first HIP call, so a rejected call
// enqueues nothing and touches no device state (and can be exercised on a
// machine without a GPU). The optional buffer checks (usp_check_buffers) are
// the exception: they query the HIP runtime about the caller's pointers, still
// before anything is enqueued.
#include <math.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "usp_common.h"
#include "usp_internal.h"

namespace {

constexpr int kAbiVersion = 121;

size_t elem_bytes(int dtype) { return dtype == USP_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const void* p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Optional checks of the caller's buffers (usp_check_buffers; initially on
// when USP_CHECK_BUFFERS is set to a value other than 0 when the library is
// first used): every span must lie inside one device (or managed) allocation
// of the current device. Off by default: each span costs two runtime queries.
// Inside a sub-allocating pool (torch's caching allocator) the allocation is
// the pool's segment, so an undersized tensor inside a segment is not caught;
// host pointers and other devices' pointers are.
std::atomic<int> g_check_buffers{-1};  // -1: the environment not read yet

bool check_buffers_on() {
  int v = g_check_buffers.load();
  if (v < 0) {
    const char* e = getenv("USP_CHECK_BUFFERS");
    const int want = (e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0')) ? 1 : 0;
    g_check_buffers.compare_exchange_strong(v, want);
    v = g_check_buffers.load();
  }
  return v == 1;
}

int check_buffer(const Span& s, int dev) {
  if (s.p == nullptr || s.n == 0) return USP_OK;
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, s.p) != hipSuccess) {
    (void)hipGetLastError();  // a failed query is not a launch error
    return USP_ERR_INVALID;
  }
  if ((at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged) || at.device != dev)
    return USP_ERR_INVALID;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(s.p)) != hipSuccess) {
    (void)hipGetLastError();
    return USP_ERR_INVALID;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), p = reinterpret_cast<uintptr_t>(s.p);
  return (p >= b && p - b <= size && s.n <= size - (p - b)) ? USP_OK : USP_ERR_INVALID;
}

// Checks the n spans at s (when the checks are on).
int check_buffers(const Span* s, int n) {
  if (!check_buffers_on()) return USP_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return USP_ERR_HIP;
  }
  for (int i = 0; i < n; ++i) {
    const int rc = check_buffer(s[i], dev);
    if (rc != USP_OK) return rc;
  }
  return USP_OK;
}

Span cu_span(const int32_t* cu, int n_docs) {
  return {cu, cu != nullptr && n_docs > 0 ? (size_t)(n_docs + 1) * 4 : 0};
}

int check_permute(const void* src, const void* dst, int64_t s_real, int p, int h, int d,
                  int dtype, size_t* src_bytes, size_t* dst_bytes, int64_t* s_pad) {
  if (dtype != USP_BF16 && dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (p < 1 || h < 1 || d < 1 || s_real < 0) return USP_ERR_INVALID;
  if (h % p != 0) return USP_ERR_INVALID;  // head count must divide the Ulysses degree
  const int64_t es = (int64_t)elem_bytes(dtype);
  const int64_t row_bytes = (int64_t)h * d * es;
  if ((row_bytes / p) % 4 != 0) return USP_ERR_UNSUPPORTED;
  *s_pad = usp_padded_len(s_real, p);
  // kernels index 4-byte chunks with 32-bit integers
  if (*s_pad > 0 && (double)(*s_pad) * (double)(row_bytes / 4) >= 2147483648.0) return USP_ERR_INVALID;
  *src_bytes = (size_t)(s_real * row_bytes);
  *dst_bytes = (size_t)(*s_pad * row_bytes);
  return USP_OK;
}

constexpr int64_t kMaxPos = (int64_t)1 << 30;  // global positions are 32-bit in the kernels

int check_heads(int hq, int hkv, int d, float scale, int causal, int dtype) {
  if (dtype != USP_BF16 && dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return USP_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return USP_ERR_INVALID;
  if (causal != 0 && causal != 1) return USP_ERR_INVALID;
  if (d != 64 && d != 128) return USP_ERR_UNSUPPORTED;
  return USP_OK;
}

int check_attn(int64_t s_pad, int64_t s_valid, const int32_t* cu, int n_docs, int hq, int hkv,
               int d, float scale, int causal, int dtype) {
  int rc = check_heads(hq, hkv, d, scale, causal, dtype);
  if (rc != USP_OK) return rc;
  if (s_pad < 1 || s_pad >= kMaxPos) return USP_ERR_INVALID;
  if (s_valid < 1 || s_valid > s_pad) return USP_ERR_INVALID;
  if (cu != nullptr && (n_docs < 1 || s_valid != s_pad)) return USP_ERR_INVALID;
  if ((double)s_pad * hq * d >= 9.0e15) return USP_ERR_INVALID;
  return USP_OK;
}

int check_interval(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off, int64_t s_k_valid,
                   const int32_t* cu, int n_docs, int hq, int hkv, int d, float scale, int causal,
                   int dtype) {
  int rc = check_heads(hq, hkv, d, scale, causal, dtype);
  if (rc != USP_OK) return rc;
  if (s_q < 1 || s_k < 1 || q_off < 0 || k_off < 0) return USP_ERR_INVALID;
  if (q_off + s_q >= kMaxPos || k_off + s_k >= kMaxPos) return USP_ERR_INVALID;
  if (s_k_valid < 0 || s_k_valid > s_k) return USP_ERR_INVALID;
  if (cu != nullptr && n_docs < 1) return USP_ERR_INVALID;
  if ((double)(s_q > s_k ? s_q : s_k) * hq * d >= 9.0e15) return USP_ERR_INVALID;
  return USP_OK;
}

// The attention call with both ends as intervals: every entry point lands here
// after its own checks.
usp::AttnArgs interval_args(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                            int64_t s_k_valid, const int32_t* cu, int n_docs, int hq, int hkv,
                            int d, float scale, int causal, void* stream) {
  usp::AttnArgs a{};
  a.s_q = s_q; a.q_off = q_off; a.s_k = s_k; a.k_off = k_off; a.s_kv = s_k_valid;
  a.lim = q_off + s_q > k_off + s_k ? q_off + s_q : k_off + s_k;
  a.cu = cu; a.n_docs = n_docs;
  a.hq = hq; a.hkv = hkv; a.d = d; a.scale = scale; a.causal = causal;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

int fwd_checked(const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes, int64_t s_q, int64_t q_off, int64_t s_k,
                int64_t k_off, int64_t s_k_valid, const int32_t* cu, int n_docs, int hq, int hkv,
                int d, float scale, int causal, int dtype, int o_dtype, void* stream) {
  if (o_dtype != USP_BF16 && o_dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (dtype == USP_FP32 && o_dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse) return USP_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return USP_ERR_INVALID;
  if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u)) return USP_ERR_INVALID;
  const size_t es = elem_bytes(dtype);
  const size_t qb = (size_t)s_q * hq * d * es, kb = (size_t)s_k * hkv * d * es;
  const size_t ob = (size_t)s_q * hq * d * elem_bytes(o_dtype);
  const size_t lb = (size_t)s_q * hq * sizeof(float);
  // bf16: the key-major V copy is required; room beyond it (as much as
  // usp_attn_fwd_workspace_bytes) lets a short call split its keys
  const size_t need = dtype == USP_BF16 ? usp::attn_fwd_bf16_min_workspace(s_k, hkv, d) : 0;
  const Span ins[] = {{q, qb}, {k, kb}, {v, kb}};
  const Span outs[] = {{o, ob}, {lse, lb}, {workspace, need > 0 ? workspace_bytes : 0}};
  // the optional buffer checks come before the workspace size check, so a
  // call with an undersized workspace exercises them without launching
  const Span all[] = {ins[0], ins[1], ins[2], outs[0], outs[1], outs[2], cu_span(cu, n_docs)};
  const int rc = check_buffers(all, 7);
  if (rc != USP_OK) return rc;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return USP_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return USP_ERR_INVALID;
  for (const Span& a : outs) {
    for (const Span& b : ins)
      if (overlap(a, b)) return USP_ERR_INVALID;
  }
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2]))
    return USP_ERR_INVALID;
  usp::AttnArgs a = interval_args(s_q, q_off, s_k, k_off, s_k_valid, cu, n_docs, hq, hkv, d,
                                  scale, causal, stream);
  a.q = q; a.k = k; a.v = v;
  a.o_out = o; a.lse_out = lse; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.out_f32 = o_dtype == USP_FP32;
  return dtype == USP_BF16 ? usp::attn_fwd_bf16(a) : usp::attn_fwd_f32(a);
}

// Every check of a backward call that does not involve the workspace; on
// success *need holds the workspace bytes the call requires and *spans the
// caller's input and output ranges.
struct BwdSpans {
  Span ins[6], outs[3];
};

int bwd_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int64_t s_q, int64_t s_k,
                 const int32_t* cu, int hq, int hkv, int d, int dtype, int grad_dtype,
                 int accumulate, size_t* need, BwdSpans* sp) {
  if (grad_dtype != USP_BF16 && grad_dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (dtype == USP_FP32 && grad_dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (accumulate != 0 && accumulate != 1) return USP_ERR_INVALID;
  if (accumulate && grad_dtype != USP_FP32) return USP_ERR_INVALID;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return USP_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return USP_ERR_INVALID;
  if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u)) return USP_ERR_INVALID;
  const size_t es = elem_bytes(dtype), gs = elem_bytes(grad_dtype);
  const size_t qb = (size_t)s_q * hq * d * es, kb = (size_t)s_k * hkv * d * es;
  const size_t gqb = (size_t)s_q * hq * d * gs, gkb = (size_t)s_k * hkv * d * gs;
  const size_t lb = (size_t)s_q * hq * sizeof(float);
  *sp = BwdSpans{{{q, qb}, {k, kb}, {v, kb}, {o, qb}, {lse, lb}, {dout, qb}},
                 {{dq, gqb}, {dk, gkb}, {dv, gkb}}};
  for (const Span& a : sp->outs)
    for (const Span& b : sp->ins)
      if (overlap(a, b)) return USP_ERR_INVALID;
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlap(sp->outs[i], sp->outs[j])) return USP_ERR_INVALID;
  // bf16: room beyond the required part (as much as the workspace query
  // returns) lets a short call split dQ's keys
  *need = dtype == USP_BF16 ? usp::attn_bwd_bf16_min_workspace(s_q, s_k, hq, hkv, d)
                            : usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, dtype);
  return USP_OK;
}

int bwd_dispatch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                 int64_t s_k_valid, const int32_t* cu, int n_docs, int hq, int hkv, int d,
                 float scale, int causal, int dtype, int grad_dtype, int accumulate,
                 void* stream) {
  usp::AttnArgs a = interval_args(s_q, q_off, s_k, k_off, s_k_valid, cu, n_docs, hq, hkv, d,
                                  scale, causal, stream);
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.out_f32 = grad_dtype == USP_FP32;
  a.accumulate = accumulate;
  return dtype == USP_BF16 ? usp::attn_bwd_bf16(a) : usp::attn_bwd_f32(a);
}

int bwd_checked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                int64_t s_k_valid, const int32_t* cu, int n_docs, int hq, int hkv, int d,
                float scale, int causal, int dtype, int grad_dtype, int accumulate, void* stream) {
  size_t need = 0;
  BwdSpans sp;
  int rc = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, s_q, s_k, cu, hq, hkv, d, dtype,
                        grad_dtype, accumulate, &need, &sp);
  if (rc != USP_OK) return rc;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return USP_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return USP_ERR_INVALID;
  const Span ws{workspace, need > 0 ? (dtype == USP_BF16 ? workspace_bytes : need) : 0};
  for (const Span& b : sp.ins)
    if (overlap(ws, b)) return USP_ERR_INVALID;
  for (const Span& b : sp.outs)
    if (overlap(ws, b)) return USP_ERR_INVALID;
  const Span all[] = {sp.ins[0], sp.ins[1],  sp.ins[2],  sp.ins[3], sp.ins[4],
                      sp.ins[5], sp.outs[0], sp.outs[1], sp.outs[2], ws, cu_span(cu, n_docs)};
  rc = check_buffers(all, 11);
  if (rc != USP_OK) return rc;
  return bwd_dispatch(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, s_q, q_off,
                      s_k, k_off, s_k_valid, cu, n_docs, hq, hkv, d, scale, causal, dtype,
                      grad_dtype, accumulate, stream);
}

// The backward workspace of usp_attn_bwd_noalloc: a library-owned array in
// device memory, one per GPU (each device that loads the library's code
// object holds its own copy at its own address), kept until the process ends.
// In host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[USP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array (looked up on first use).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return USP_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return USP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return USP_OK;
}

}  // namespace

extern "C" {

int usp_version(void) { return kAbiVersion; }

int usp_check_buffers(int on) {
  const int prev = check_buffers_on() ? 1 : 0;
  if (on >= 0) g_check_buffers.store(on ? 1 : 0);
  return prev;
}

const char* usp_status_string(int status) {
  switch (status) {
    case USP_OK: return "ok";
    case USP_ERR_INVALID: return "invalid argument (shape, divisibility, range, alignment or aliasing)";
    case USP_ERR_UNSUPPORTED: return "unsupported dtype or head dimension";
    case USP_ERR_NULL: return "required pointer is NULL";
    case USP_ERR_HIP: return "HIP runtime error while launching";
    case USP_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int64_t usp_padded_len(int64_t s_real, int p) {
  if (p < 1 || s_real < 0) return -1;
  return (s_real + p - 1) / p * p;
}

static int permute_entry(bool pack, const void* src, void* dst, int64_t s_real, int p, int h,
                         int d, int dtype, void* stream) {
  size_t src_bytes = 0, dst_bytes = 0;
  int64_t s_pad = 0;
  const int64_t s_rows = s_real;
  // for the pack src is x [s_real][h][d]; for the unpack src is y [p][s_pad][h/p][d]
  int rc = check_permute(src, dst, s_rows, p, h, d, dtype, &src_bytes, &dst_bytes, &s_pad);
  if (rc != USP_OK) return rc;
  const size_t x_bytes = src_bytes, y_bytes = dst_bytes;
  const size_t in_bytes = pack ? x_bytes : y_bytes;
  const size_t out_bytes = pack ? y_bytes : x_bytes;
  if (out_bytes == 0) return USP_OK;
  if ((in_bytes > 0 && src == nullptr) || dst == nullptr) return USP_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return USP_ERR_INVALID;
  if (overlap({src, in_bytes}, {dst, out_bytes})) return USP_ERR_INVALID;
  const Span all[] = {{src, in_bytes}, {dst, out_bytes}};
  rc = check_buffers(all, 2);
  if (rc != USP_OK) return rc;
  const int64_t row_bytes = (int64_t)h * d * (int64_t)elem_bytes(dtype);
  return usp::permute_launch(pack, src, dst, s_real, s_pad, p, row_bytes,
                             static_cast<hipStream_t>(stream));
}

int usp_pad_pack_seq2head(const void* x, void* y, int64_t s_real, int p, int h, int d, int dtype,
                          void* stream) {
  return permute_entry(true, x, y, s_real, p, h, d, dtype, stream);
}

int usp_unpack_head2seq(const void* y, void* x, int64_t s_real, int p, int h, int d, int dtype,
                        void* stream) {
  return permute_entry(false, y, x, s_real, p, h, d, dtype, stream);
}

size_t usp_attn_fwd_workspace_bytes(int64_t s_pad, int hq, int hkv, int d, int dtype) {
  if (s_pad < 1 || hq < 1 || hkv < 1 || d < 1) return 0;
  if (dtype == USP_BF16) return usp::attn_fwd_bf16_workspace(s_pad, hq, hkv, d);
  return 0;
}

size_t usp_attn_bwd_interval_workspace_bytes(int64_t s_q, int64_t s_k, int hq, int hkv, int d,
                                             int dtype) {
  if (s_q < 1 || s_k < 1 || hq < 1 || hkv < 1 || d < 1) return 0;
  if (dtype == USP_BF16) return usp::attn_bwd_bf16_workspace(s_q, s_k, hq, hkv, d);
  return usp::attn_bwd_f32_workspace(s_q, hq, hkv, d);
}

size_t usp_attn_bwd_workspace_bytes(int64_t s_pad, int hq, int hkv, int d, int dtype) {
  return usp_attn_bwd_interval_workspace_bytes(s_pad, s_pad, hq, hkv, d, dtype);
}

int usp_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, int64_t s_pad, int64_t s_valid,
                 const int32_t* cu_seqlens, int n_docs, int hq, int hkv, int d,
                 float softmax_scale, int causal, int dtype, void* stream) {
  int rc = check_attn(s_pad, s_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal, dtype);
  if (rc != USP_OK) return rc;
  return fwd_checked(q, k, v, o, lse, workspace, workspace_bytes, s_pad, 0, s_pad, 0, s_valid,
                     cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal, dtype, dtype, stream);
}

int usp_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int64_t s_pad, int64_t s_valid,
                 const int32_t* cu_seqlens, int n_docs, int hq, int hkv, int d,
                 float softmax_scale, int causal, int dtype, void* stream) {
  int rc = check_attn(s_pad, s_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal, dtype);
  if (rc != USP_OK) return rc;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, s_pad, 0,
                     s_pad, 0, s_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal,
                     dtype, dtype, 0, stream);
}

int usp_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         int64_t s_pad, int64_t s_valid, const int32_t* cu_seqlens, int n_docs,
                         int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                         void* stream) {
  int rc = check_attn(s_pad, s_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal, dtype);
  if (rc != USP_OK) return rc;
  size_t need = 0;
  BwdSpans sp;
  rc = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, s_pad, s_pad, cu_seqlens, hq, hkv, d, dtype,
                    dtype, 0, &need, &sp);
  if (rc != USP_OK) return rc;
  if (need > (size_t)USP_NOALLOC_SCRATCH_BYTES) return USP_ERR_WORKSPACE;
  const Span all[] = {sp.ins[0], sp.ins[1],  sp.ins[2],  sp.ins[3],  sp.ins[4],
                      sp.ins[5], sp.outs[0], sp.outs[1], sp.outs[2], cu_span(cu_seqlens, n_docs)};
  rc = check_buffers(all, 10);
  if (rc != USP_OK) return rc;
  // the first HIP call of the dispatch: every argument check has passed
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != USP_OK) return rc;
  return bwd_dispatch(q, k, v, o, lse, dout, dq, dk, dv, ws, USP_NOALLOC_SCRATCH_BYTES, s_pad, 0,
                      s_pad, 0, s_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal,
                      dtype, dtype, 0, stream);
}

int usp_attn_fwd_interval(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int64_t s_q, int64_t q_off,
                          int64_t s_k, int64_t k_off, int64_t s_k_valid,
                          const int32_t* cu_seqlens, int n_docs, int hq, int hkv, int d,
                          float softmax_scale, int causal, int dtype, int o_dtype, void* stream) {
  int rc = check_interval(s_q, q_off, s_k, k_off, s_k_valid, cu_seqlens, n_docs, hq, hkv, d,
                          softmax_scale, causal, dtype);
  if (rc != USP_OK) return rc;
  return fwd_checked(q, k, v, o, lse, workspace, workspace_bytes, s_q, q_off, s_k, k_off,
                     s_k_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal, dtype,
                     o_dtype, stream);
}

int usp_attn_fwd_num_splits(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                            int64_t s_k_valid, int hq, int hkv, int d, int causal, int dtype,
                            size_t workspace_bytes) {
  const int rc = check_interval(s_q, q_off, s_k, k_off, s_k_valid, nullptr, 0, hq, hkv, d, 1.0f,
                                causal, dtype);
  if (rc != USP_OK) return rc;
  if (dtype != USP_BF16) return 1;
  usp::AttnArgs a = interval_args(s_q, q_off, s_k, k_off, s_k_valid, nullptr, 0, hq, hkv, d, 1.0f,
                                  causal, nullptr);
  a.workspace_bytes = workspace_bytes;
  return usp::attn_fwd_bf16_splits(a);
}

int usp_attn_bwd_num_splits(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                            int64_t s_k_valid, int hq, int hkv, int d, int causal, int dtype,
                            size_t workspace_bytes) {
  const int rc = check_interval(s_q, q_off, s_k, k_off, s_k_valid, nullptr, 0, hq, hkv, d, 1.0f,
                                causal, dtype);
  if (rc != USP_OK) return rc;
  if (dtype != USP_BF16) return 1;
  usp::AttnArgs a = interval_args(s_q, q_off, s_k, k_off, s_k_valid, nullptr, 0, hq, hkv, d, 1.0f,
                                  causal, nullptr);
  a.workspace_bytes = workspace_bytes;
  return usp::attn_bwd_bf16_dq_splits(a);
}

int usp_attn_bwd_interval(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int64_t s_q, int64_t q_off,
                          int64_t s_k, int64_t k_off, int64_t s_k_valid,
                          const int32_t* cu_seqlens, int n_docs, int hq, int hkv, int d,
                          float softmax_scale, int causal, int dtype, int grad_dtype,
                          int accumulate, void* stream) {
  int rc = check_interval(s_q, q_off, s_k, k_off, s_k_valid, cu_seqlens, n_docs, hq, hkv, d,
                          softmax_scale, causal, dtype);
  if (rc != USP_OK) return rc;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, s_q, q_off,
                     s_k, k_off, s_k_valid, cu_seqlens, n_docs, hq, hkv, d, softmax_scale, causal,
                     dtype, grad_dtype, accumulate, stream);
}

int usp_attn_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                   void* o, float* lse, int64_t s_q, int hq, int d, int o_dtype, void* stream) {
  if (o_dtype != USP_BF16 && o_dtype != USP_FP32) return USP_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return USP_ERR_UNSUPPORTED;
  if (s_q < 1 || hq < 1 || (double)s_q * hq * d >= 2147483648.0) return USP_ERR_INVALID;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return USP_ERR_NULL;
  const void* ptrs[] = {o_a, lse_a, o_b, lse_b, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return USP_ERR_INVALID;
  const size_t ob = (size_t)s_q * hq * d * 4, lb = (size_t)s_q * hq * 4;
  const size_t oob = (size_t)s_q * hq * d * elem_bytes(o_dtype);
  // the outputs may BE an input (in-place accumulation), never partly overlap one
  const Span o_ins[] = {{o_a, ob}, {o_b, ob}, {lse_a, lb}, {lse_b, lb}};
  for (const Span& b : o_ins) {
    const bool same = b.p == o && b.n == oob && (b.p == o_a || b.p == o_b);
    if (!same && overlap({o, oob}, b)) return USP_ERR_INVALID;
  }
  for (const Span& b : o_ins) {
    const bool same = b.p == lse && (b.p == lse_a || b.p == lse_b);
    if (!same && overlap({lse, lb}, b)) return USP_ERR_INVALID;
  }
  if (overlap({o, oob}, {lse, lb})) return USP_ERR_INVALID;
  const Span all[] = {o_ins[0], o_ins[1], o_ins[2], o_ins[3], {o, oob}, {lse, lb}};
  const int rc = check_buffers(all, 6);
  if (rc != USP_OK) return rc;
  return usp::attn_merge_launch(o_a, lse_a, o_b, lse_b, o, lse, s_q, hq, d,
                                o_dtype == USP_FP32, static_cast<hipStream_t>(stream));
}

}  // extern "C"
