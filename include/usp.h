/*
 * usp.h: C ABI of the Ulysses sequence-parallel rank-share hot path on
 * MI355X (gfx950).
 *
 * What the calls compute. In Ulysses sequence parallelism each of P ranks
 * holds one contiguous slice of the (padded) sequence with all heads. Separate
 * all-to-alls of Q, K and V give every rank the full sequence restricted to its
 * H/P heads; it runs ordinary attention locally and a reverse all-to-all returns
 * the output to sequence slices ("feat(dspark): add Ulysses sequence parallel
 * training", Motivation and Modifications: shard-and-pad, separate Q/K/V
 * all-to-alls, head counts divisible by the Ulysses degree). On one device the
 * P packs plus the all-to-all compose into usp_pad_pack_seq2head, the reverse
 * into usp_unpack_head2seq, and usp_attn_fwd / usp_attn_bwd are one rank's
 * local attention, forward and backward (same page, Accuracy Test: loss and
 * gradient parity with full-sequence attention), with packed documents given by
 * cu_seqlens ("GLM-5.2 131k context parallelism", Purpose: THD packed
 * sequences).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE memory of the current device, owned by
 *     the caller; the library never allocates device memory and keeps no state
 *     between calls (apart from the optional kernel trace below and the static
 *     workspace array of usp_attn_bwd_noalloc). The library cannot tell a host
 *     pointer or another device's pointer from a valid one: passing one is
 *     undefined (the kernels would access it). The Python binding refuses such
 *     tensors before the call.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t of the current
 *     device passed as void*; NULL means the default stream). The return value is known
 *     synchronously: argument checks run on the host before any HIP call, so a
 *     rejected call enqueues nothing.
 *   - Tensor pointers must be 16-byte aligned; outputs may not overlap inputs.
 *   - dtype is USP_BF16 (bfloat16 storage, fp32 accumulation) or USP_FP32.
 *   - Errors are return codes only (usp_status); usp_status_string() names them.
 */
#ifndef USP_H_
#define USP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  USP_OK = 0,
  USP_ERR_INVALID = -1,     /* shape, divisibility, range, alignment or aliasing */
  USP_ERR_UNSUPPORTED = -2, /* dtype / head dim not built */
  USP_ERR_NULL = -3,        /* a required pointer is NULL */
  USP_ERR_HIP = -4,         /* the HIP runtime reported a launch error */
  USP_ERR_WORKSPACE = -5    /* workspace NULL or smaller than required */
} usp_status;

typedef enum { USP_BF16 = 0, USP_FP32 = 1 } usp_dtype;

/* Library ABI version (major*100 + minor). */
int usp_version(void);

/* Human-readable name of a usp_status value (static string, never NULL). */
const char* usp_status_string(int status);

/*
 * Optional checks of the caller's buffers, for debugging. When on, every call
 * first asks the HIP runtime about each tensor it is given (its byte range
 * from the shapes): the range must lie inside one device or managed allocation
 * of the current device, or the call returns USP_ERR_INVALID and enqueues
 * nothing. Catches host pointers, another device's pointers and buffers
 * smaller than their shape inside a plain hipMalloc allocation; inside a pool
 * that sub-allocates (such as torch's caching allocator) the allocation is the
 * pool's segment, so only ranges that leave the segment are caught. Off by
 * default (two runtime queries per tensor); initially on when the environment
 * variable USP_CHECK_BUFFERS is set to anything but "0" at the library's first
 * use.
 *   on: 1 turns the checks on, 0 off, a negative value leaves them as they are.
 * Returns the previous state (1 on, 0 off). Thread-safe; affects calls that
 * start after it returns.
 */
int usp_check_buffers(int on);

/*
 * Padded sequence length for a Ulysses degree p: the smallest multiple of p
 * that is >= s_real (alignment padding before sharding, "feat(dspark)",
 * Modifications). Returns -1 if p < 1 or s_real < 0.
 */
int64_t usp_padded_len(int64_t s_real, int p);

/*
 * Pad + pack, sequence-sharded -> head-sharded ("feat(dspark)", Modifications:
 * shard and pad, then the Q/K/V all-to-all). With hp = h / p and
 * s_pad = usp_padded_len(s_real, p):
 *     y[r][s][j][:] = x[s][r*hp + j][:]   for s <  s_real
 *     y[r][s][j][:] = 0                   for s_real <= s < s_pad
 *   x: [s_real][h][d] row-major, read only.
 *   y: [p][s_pad][hp][d] row-major, fully overwritten (padding rows included).
 * Bit-exact copy. Errors: USP_ERR_INVALID if h % p != 0, p < 1, h < 1, d < 1,
 * s_real < 0, misaligned pointers, or overlap of x and y; USP_ERR_UNSUPPORTED
 * if d * sizeof(elem) is not a multiple of 4 bytes; USP_ERR_NULL for NULL
 * pointers when there is data. s_real = 0 writes nothing.
 */
int usp_pad_pack_seq2head(const void* x, void* y, int64_t s_real, int p, int h, int d,
                          int dtype, void* stream);

/*
 * Unpack, head-sharded -> sequence-sharded: the inverse of the pack on the real
 * rows, padding rows dropped (the reverse all-to-all that returns the attention
 * output to each rank's slice).
 *     x[s][r*hp + j][:] = y[r][s][j][:]   for s < s_real
 *   y: [p][s_pad][hp][d] read only; x: [s_real][h][d] fully overwritten.
 * Same errors as the pack.
 */
int usp_unpack_head2seq(const void* y, void* x, int64_t s_real, int p, int h, int d,
                        int dtype, void* stream);

/*
 * Workspace bytes usp_attn_fwd needs (0 for USP_FP32). The bf16 path stores a
 * key-major copy of V there and, when s_pad rows make a grid of fewer than 512
 * workgroups (short sequences), room for up to 8 key splits: fp32 partial O
 * and LSE of every query row, combined exactly by a merge kernel (see
 * usp_attn_fwd_num_splits). The room is for min(8, ceil(1024 / workgroups))
 * splits: about 135 MB at s_pad = 8192 with 4 query heads, one KV head and
 * d = 128 (8 splits) or at 16,384 (4 splits); none from 32,768 rows per KV
 * head at 4:1 GQA upwards. Without splits the room holds a small table
 * instead (12 bytes per block of query rows, 256-byte aligned): a call with
 * cu_seqlens runs its query blocks longest first, an order two small kernels
 * compute from the documents (within one document the work of a block grows
 * with its position; the natural order, last block first, is longest first
 * only for a single sequence). The order only schedules the same per-block
 * arithmetic: outputs are bit for bit those of the natural order, which a
 * call without room for the table keeps.
 */
size_t usp_attn_fwd_workspace_bytes(int64_t s_pad, int hq, int hkv, int d, int dtype);

/*
 * Attention forward over one rank's share: the full (padded) sequence, hq query
 * heads, hkv key/value heads, query head i reading key/value head i / (hq/hkv).
 * For query row i the allowed keys are
 *     M(i) = { j < s_valid, doc(j) == doc(i), and j <= i when causal }
 * with doc() from cu_seqlens (one document when cu_seqlens is NULL). Then
 *     lse[h][i] = log sum_{j in M(i)} exp(scale * q_i . k_j)   (natural log)
 *     o[i][h]   = sum_{j in M(i)} exp(scale * q_i . k_j - lse[h][i]) v_j
 * Padded query rows (i >= s_valid) are computed like any other row.
 *   q: [s_pad][hq][d], k and v: [s_pad][hkv][d], read only.
 *   o: [s_pad][hq][d] (dtype), lse: [hq][s_pad] fp32; both fully overwritten.
 *   cu_seqlens: device int32 [n_docs + 1] with 0 = cu[0] <= ... <= cu[n_docs]
 *     = s_pad, or NULL. Its contents are not checked (device memory); values
 *     outside [0, s_pad] are clamped, never dereferenced out of range.
 *   workspace: device memory of usp_attn_fwd_workspace_bytes() bytes (may be
 *     NULL when that is 0); contents are scratch. For bf16 the V copy,
 *     hkv * d * round_up(s_pad, 128) * 2 bytes, is the minimum; with less room
 *     than the query returns the call runs fewer key splits (one pass with
 *     none), same results up to rounding. The whole workspace_bytes range must
 *     not overlap the other arguments.
 * Supported: d in {64, 128}, both dtypes.
 * Errors: USP_ERR_INVALID for s_valid < 1 or > s_pad, hq % hkv != 0,
 * cu_seqlens with s_valid != s_pad or n_docs < 1, misalignment, aliasing;
 * USP_ERR_UNSUPPORTED for other d / dtype; USP_ERR_WORKSPACE if the workspace
 * is too small.
 */
int usp_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes,
                 int64_t s_pad, int64_t s_valid, const int32_t* cu_seqlens, int n_docs,
                 int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                 void* stream);

/* Workspace bytes usp_attn_bwd needs for these sizes: per (query head, row)
 * fp32 D and LSE values and, for bf16 on short sequences (one KV head: fewer
 * than 512 blocks of 128 keys, up to 16 row chunks; several KV heads: fewer
 * than 1024 (block, KV head) pairs, 2 row chunks), fp32 partial dK and dV per
 * row chunk; deterministic in the sizes. That much is required. For bf16 the
 * size returned also holds room for up to 8 key splits of dQ when the dQ grid
 * has fewer than 1024 workgroups (fp32 partial dQ of every row, summed in a
 * fixed order afterwards; see usp_attn_bwd_num_splits): about 134 MB at
 * s_pad = 8192 with 4 query heads and d = 128. With less room the call splits
 * less (one pass with none), same results up to rounding. Without splits or
 * row chunks the room holds two small tables instead (12 bytes per block of
 * 128 keys and per dQ block of query rows), with which a call with
 * cu_seqlens runs both kernels' blocks longest first, as usp_attn_fwd does
 * (same outputs bit for bit). The whole workspace_bytes range must not
 * overlap the other arguments. */
size_t usp_attn_bwd_workspace_bytes(int64_t s_pad, int hq, int hkv, int d, int dtype);

/*
 * Attention backward for the loss whose gradient with respect to o is dout
 * (chain rule through the softmax; gradient parity in "feat(dspark)", Accuracy
 * Test). With P_ij = exp(scale q_i.k_j - lse_i) on M(i), dP_ij = dout_i . v_j,
 * D_i = sum_j P_ij dP_ij (taken as dout_i . o_i) and dS = P (dP - D):
 *     dq_i = scale sum_j dS_ij k_j
 *     dk_j = scale sum_{heads of the group} sum_i dS_ij q_i
 *     dv_j = sum_{heads of the group} sum_i P_ij dout_i
 *   q, o, dout: [s_pad][hq][d]; k, v: [s_pad][hkv][d]; lse: [hq][s_pad] fp32
 *     as written by usp_attn_fwd; all read only.
 *   dq: [s_pad][hq][d], dk and dv: [s_pad][hkv][d]; fully overwritten.
 *   workspace: usp_attn_bwd_workspace_bytes() bytes of device scratch.
 * Masks, supported sizes and errors as in usp_attn_fwd.
 */
int usp_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int64_t s_pad, int64_t s_valid, const int32_t* cu_seqlens, int n_docs,
                 int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                 void* stream);

/* Size of the library-owned backward workspace of usp_attn_bwd_noalloc, per
 * GPU: 32 MiB. */
#define USP_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * usp_attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same computation, kernels, arguments, outputs and
 * errors as usp_attn_bwd; the workspace is a library-owned array of
 * USP_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, which each GPU the
 * call runs on holds until the process ends. The call allocates nothing
 * (no hipMalloc, no allocating library routine).
 *   - The array of the CURRENT device is used: stream must belong to it.
 *   - Calls on one GPU share its array. Calls that may overlap in time on one
 *     GPU (different streams without ordering between them) race on it and
 *     must not be issued; calls ordered on one stream are fine. Each call
 *     rewrites every part of the array it reads, so nothing carries over from
 *     the previous call and nothing needs clearing.
 *   - Sizes whose required workspace (usp_attn_bwd's minimum: fp32 D and LSE
 *     per query row and head, plus the dK/dV row-chunk partials of short
 *     sequences) exceeds USP_NOALLOC_SCRATCH_BYTES return USP_ERR_WORKSPACE
 *     before any device work: for example 120,000 rows with 4 query heads
 *     need 3.8 MB and 131,072 rows with 16 heads 16.8 MB, but 8,192 rows on
 *     one KV head (16 row chunks, 134 MB) are rejected. Room left in the array
 *     goes to dQ key splits, or to the longest-first block order of calls
 *     with cu_seqlens, as in usp_attn_bwd.
 */
int usp_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         int64_t s_pad, int64_t s_valid, const int32_t* cu_seqlens, int n_docs,
                         int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                         void* stream);

/*
 * Attention between a query interval and a key interval on global positions:
 * the partial result of one ring step of Ring / USP attention (the ring degree
 * of USP: "feat(dspark)", Accuracy Test; "[trainer] feat: support sequence
 * parallel", review overview, the (dp, ring, ulysses) device mesh), or a
 * contiguous context-parallel rank's query rows against the whole key sequence
 * with a causal offset ("GLM-5.2 131k context parallelism", Purpose: causal
 * query offsets and positions from global cu_seqlens over each rank's
 * contiguous row interval).
 * Query row i sits at global position q_off + i (i < s_q), key j at k_off + j
 * (j < s_k). The allowed keys of row i are
 *     M(i) = { j < s_k_valid, doc(k_off + j) == doc(q_off + i), and
 *              k_off + j <= q_off + i when causal }
 * with doc() from cu_seqlens over GLOBAL positions (one document when NULL).
 * Then, as in usp_attn_fwd, lse[h][i] = log sum_{j in M(i)} exp(scale q_i.k_j)
 * and o[i][h] = sum_{j in M(i)} exp(scale q_i.k_j - lse[h][i]) v_j; a row with
 * M(i) empty gets o = 0 and lse = -inf (the identity of usp_attn_merge).
 * usp_attn_fwd(...) equals this call with s_q = s_k = s_pad, q_off = k_off = 0.
 *   q: [s_q][hq][d], k and v: [s_k][hkv][d] (dtype), read only.
 *   o: [s_q][hq][d] in o_dtype (USP_FP32 for a partial that will be merged,
 *     USP_BF16 allowed for bf16 inputs); lse: [hq][s_q] fp32. Both overwritten.
 *   cu_seqlens: device int32 [n_docs + 1], 0 = cu[0] <= ... <= cu[n_docs], and
 *     cu[n_docs] >= q_off + s_q and >= k_off + s_k; or NULL. Not checked.
 *   workspace: usp_attn_fwd_workspace_bytes(s_k, hq, hkv, d, dtype) bytes, at
 *     least the V copy as in usp_attn_fwd (room for the key splits of s_q rows
 *     when s_q > s_k may need more; with less the call splits less).
 * Errors: USP_ERR_INVALID for s_q < 1, s_k < 1, negative offsets,
 * q_off + s_q or k_off + s_k >= 2^30, s_k_valid outside [0, s_k], the head and
 * scale checks of usp_attn_fwd, misalignment or aliasing; USP_ERR_UNSUPPORTED
 * for d / dtype as in usp_attn_fwd, or o_dtype USP_BF16 with fp32 inputs.
 */
int usp_attn_fwd_interval(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                          int64_t s_k_valid, const int32_t* cu_seqlens, int n_docs,
                          int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                          int o_dtype, void* stream);

/*
 * Number of key splits usp_attn_fwd / usp_attn_fwd_interval run for these
 * arguments with a workspace of workspace_bytes bytes (1: a single pass).
 * With n > 1 splits each query block's key tiles are cut into n consecutive
 * ranges processed by separate workgroups (so a short sequence fills the
 * chip and the long rows of the causal triangle are shared out); each writes
 * an fp32 partial O and LSE into the workspace and a merge kernel combines
 * them exactly (the identity of usp_attn_merge), then writes o and lse. The
 * plan depends only on these arguments (not on cu_seqlens' contents or the
 * data), so a call is deterministic. Host-only: no device is touched.
 * Returns the count, or the error usp_attn_fwd_interval would return for
 * these sizes (USP_ERR_INVALID, USP_ERR_UNSUPPORTED).
 */
int usp_attn_fwd_num_splits(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                            int64_t s_k_valid, int hq, int hkv, int d, int causal, int dtype,
                            size_t workspace_bytes);

/*
 * Number of key splits the dQ kernel of usp_attn_bwd / usp_attn_bwd_interval
 * runs for these arguments with a workspace of workspace_bytes bytes (1: a
 * single pass). With n > 1 each block of query rows has its key tiles cut
 * into n consecutive ranges run by separate workgroups, each writing an fp32
 * partial dQ into the workspace; a reduction kernel adds them in split order
 * (deterministic) and writes dq (or adds to it when accumulating). dK and dV
 * are unaffected. Like usp_attn_fwd_num_splits, host-only and independent of
 * cu_seqlens' contents and the data. Returns the count or the error the call
 * would return for these sizes.
 */
int usp_attn_bwd_num_splits(int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                            int64_t s_k_valid, int hq, int hkv, int d, int causal, int dtype,
                            size_t workspace_bytes);

/*
 * Exact merge of two partial results over disjoint key sets of the same query
 * rows (combining the ring steps of Ring / USP attention; same sources as
 * usp_attn_fwd_interval):
 *     lse = log(exp(lse_a) + exp(lse_b))
 *     o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
 * Rows with lse_a = lse_b = -inf give o = 0, lse = -inf.
 *   o_a, o_b: [s_q][hq][d] fp32; lse_a, lse_b: [hq][s_q] fp32; read only.
 *   o: [s_q][hq][d] in o_dtype; lse: [hq][s_q] fp32; overwritten. For in-place
 *     accumulation o may BE o_a or o_b (same pointer, o_dtype USP_FP32) and lse
 *     may BE lse_a or lse_b; any other overlap is rejected.
 * Supported: d in {64, 128}. Errors: USP_ERR_INVALID for s_q < 1, hq < 1,
 * s_q * hq * d >= 2^31, misalignment or partial overlap; USP_ERR_UNSUPPORTED
 * for other d or o_dtype; USP_ERR_NULL for NULL pointers.
 */
int usp_attn_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                   void* o, float* lse, int64_t s_q, int hq, int d, int o_dtype, void* stream);

/* Workspace bytes usp_attn_bwd_interval needs for these sizes (as for
 * usp_attn_bwd, with s_q query rows and s_k keys). */
size_t usp_attn_bwd_interval_workspace_bytes(int64_t s_q, int64_t s_k, int hq, int hkv, int d,
                                             int dtype);

/*
 * Backward of one (query interval, key interval) pair, given the FINAL output o
 * and the FINAL (merged) lse of the query rows: the pair's contributions
 *     dq_i = scale sum_{j in M(i)} dS_ij k_j
 *     dk_j = scale sum_{heads of the group} sum_i dS_ij q_i
 *     dv_j = sum_{heads of the group} sum_i P_ij dout_i
 * with M(i), P, dP, D = dout_i . o_i and dS = P (dP - D) as in usp_attn_bwd and
 * usp_attn_fwd_interval. Summing dq over the key intervals of a row and dk, dv
 * over the query intervals of a key gives the full gradients (the gradient
 * parity of "feat(dspark)", Accuracy Test, carried over to the ring steps).
 * usp_attn_bwd(...) equals this call with full intervals and accumulate = 0.
 *   q, o, dout: [s_q][hq][d]; k, v: [s_k][hkv][d] (dtype); lse: [hq][s_q] fp32.
 *   dq: [s_q][hq][d]; dk, dv: [s_k][hkv][d]; in grad_dtype. With accumulate = 1
 *     (grad_dtype USP_FP32 only) the contributions are ADDED to the existing
 *     contents, else they overwrite them.
 *   workspace: usp_attn_bwd_interval_workspace_bytes() bytes of scratch.
 * Errors as usp_attn_fwd_interval; USP_ERR_INVALID also for accumulate not in
 * {0, 1} or accumulate with bf16 gradients.
 */
int usp_attn_bwd_interval(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes,
                          int64_t s_q, int64_t q_off, int64_t s_k, int64_t k_off,
                          int64_t s_k_valid, const int32_t* cu_seqlens, int n_docs,
                          int hq, int hkv, int d, float softmax_scale, int causal, int dtype,
                          int grad_dtype, int accumulate, void* stream);

/*
 * Kernel tracing (profiling aid, off by default). While enabled, every kernel
 * the library launches is bracketed by a pair of HIP events recorded on its
 * stream. usp_trace_collect() waits for the recorded events, returns per-kernel
 * launch counts and summed durations (at most max_entries kernels, sorted by
 * total time, descending), and clears the record. This is the only state the
 * library keeps between calls.
 *   usp_trace_enable returns the previous setting.
 *   usp_trace_collect returns the number of entries written, or USP_ERR_NULL /
 *   USP_ERR_HIP.
 */
typedef struct {
  char name[48];
  long long launches;
  double total_ms;
} usp_trace_entry;

int usp_trace_enable(int on);
int usp_trace_collect(usp_trace_entry* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* USP_H_ */
