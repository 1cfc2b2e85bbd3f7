"""GPU parity of usp_attn_fwd / usp_attn_bwd against the fp64 oracle.

Small problems (several tiles plus a ragged tail) and an 8K-token problem on
every kernel's long-sequence path are compared element by element over every
output; the full-size workloads are compared on sampled query rows (O, LSE,
dQ), on the same sample as key rows (dK, dV, against oracle values stored by
tests/golden/make_full_size_keys.py), and through identities that hold at
any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import check_close, f64, gpu, rounding_bound, say

pytestmark = pytest.mark.gpu


def usp():
    import ulysses_sequence_parallelism_amd as m
    return m


def seeded(shape, seed, dtype):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))
    return x.to(dtype)


def run_pair(q, k, v, do, s_valid, cu, causal, dev, backward=True):
    L = usp()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = L.usp_attn_fwd(qd, kd, vd, s_valid=s_valid, cu_seqlens=cu, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = L.usp_attn_bwd(qd, kd, vd, o, lse, dod, s_valid=s_valid, cu_seqlens=cu,
                                    causal=causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


SMALL = [
    # name, S, s_valid, hq, hkv, cu_seqlens, causal
    ("one_tile", 64, 64, 4, 1, None, True),
    ("ragged", 300, 300, 4, 1, None, True),
    ("padded", 1000, 997, 4, 1, None, True),
    ("two_kv_heads", 777, 777, 8, 2, None, True),
    ("mha", 513, 513, 2, 2, None, True),
    ("gqa2", 400, 400, 4, 2, None, True),
    ("docs", 2100, 2100, 4, 1, [0, 100, 101, 1000, 1377, 2100], True),
    ("docs_16q4kv", 2048, 2048, 16, 4, [0, 700, 1300, 2048], True),
    ("bidirectional_padded", 500, 490, 4, 1, None, False),
    # no padding, length not a multiple of the 128-key block: the last block's
    # tail keys lie past the sequence end without being padding keys
    ("bidirectional_ragged", 500, 500, 4, 1, None, False),
    ("d64_bidirectional_ragged_gqa8", 2500, 2500, 8, 1, None, False, 64),
    ("bidirectional_docs", 600, 600, 4, 2, [0, 250, 600], False),
    # shorter than one 32-row block: every tile is a ragged tail
    ("tiny_1", 1, 1, 4, 1, None, True),
    ("tiny_17", 17, 17, 4, 1, None, True),
    ("tiny_bidir_33", 33, 30, 4, 2, None, False),
    # 8 query heads per KV head: two head chunks per KV head
    ("gqa8", 300, 300, 8, 1, None, True),
    # 3 query heads per KV head: one head per workgroup (256 rows), three head
    # chunks per KV head
    ("gqa3_6q2kv", 700, 700, 6, 2, None, True),
    # 16 query heads per KV head: four head chunks per KV head, padded keys
    ("gqa16_padded", 600, 590, 16, 1, None, True),
    # head dim 64 (128-byte rows: their own tile swizzle and load mapping)
    ("d64_ragged", 300, 300, 4, 1, None, True, 64),
    ("d64_padded_gqa2", 1000, 997, 4, 2, None, True, 64),
    ("d64_mha", 513, 513, 2, 2, None, True, 64),
    ("d64_docs", 2100, 2100, 4, 1, [0, 100, 101, 1000, 1377, 2100], True, 64),
    ("d64_bidir_padded", 500, 490, 8, 2, None, False, 64),
    ("d64_tiny_17", 17, 17, 4, 1, None, True, 64),
    # several KV heads at a size where every kernel runs a full grid
    ("w8_ragged_16q4kv", 4100, 4100, 16, 4, None, True),
    ("w8_docs_16q4kv", 4500, 4500, 16, 4, [0, 1000, 1001, 3000, 4500], True),
    ("w8_bidir_padded_16q4kv", 4160, 4150, 16, 4, None, False),
    ("w8_d64_16q4kv", 4100, 4100, 16, 4, None, True, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bf16_small_full_compare(case):
    name, s, s_valid, hq, hkv, cu, causal = case[:7]
    d = case[7] if len(case) > 7 else 128
    dev = gpu()
    say(f"bf16 {name}: S={s} s_valid={s_valid} hq={hq} hkv={hkv} d={d} causal={causal}")
    q, k, v, do = (seeded((s, h, d), 1000 + i, torch.bfloat16)
                   for i, h in enumerate((hq, hkv, hkv, hq)))
    if s_valid < s:  # pack zero-fills padded rows
        for t in (q, k, v, do):
            t[s_valid:] = 0
    got = run_pair(q, k, v, do, s_valid, cu, causal, dev)
    q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))
    scale = d ** -0.5
    o, lse = oracle.attn_fwd(q64, k64, v64, scale, s_valid, cu, causal)
    dq, dk, dv = oracle.attn_bwd(q64, k64, v64, o, lse, do64, scale, s_valid, cu, causal)
    check_close("O", f64(got["o"]), o, "bf16")
    check_close("LSE", f64(got["lse"]), lse, "bf16")
    check_close("dQ", f64(got["dq"]), dq, "bf16")
    check_close("dK", f64(got["dk"]), dk, "bf16")
    check_close("dV", f64(got["dv"]), dv, "bf16")


def test_fp32_tiny_sequence_parallel_pipeline():
    """The tiny fp32 workload end to end on the GPU: pack Q, K, V, dO of the
    full 8Q/4KV model for P=2, attention forward and backward on each rank's
    share, unpack O, dQ, dK, dV; compare with full-model oracle attention."""
    L = usp()
    dev = gpu()
    w = workloads.WORKLOADS["tiny"]
    xs = [workloads.tensor(w, t) for t in (workloads.Q, workloads.K, workloads.V, workloads.DO)]
    ys = [L.usp_pad_pack_seq2head(x.to(dev), w.p) for x in xs]
    outs = {n: [] for n in ("o", "dq", "dk", "dv")}
    lses = []
    for r in range(w.p):
        q, k, v, do = (y[r].contiguous() for y in ys)
        o, lse = L.usp_attn_fwd(q, k, v, softmax_scale=w.scale)
        dq, dk, dv = L.usp_attn_bwd(q, k, v, o, lse, do, softmax_scale=w.scale)
        for n, a in zip(("o", "dq", "dk", "dv"), (o, dq, dk, dv)):
            outs[n].append(a)
        lses.append(lse)
    got = {n: L.usp_unpack_head2seq(torch.stack(a).contiguous(), w.s) for n, a in outs.items()}
    torch.cuda.synchronize()
    x64 = [f64(x) for x in xs]
    o, lse = oracle.attn_fwd(x64[0], x64[1], x64[2], w.scale)
    dq, dk, dv = oracle.attn_bwd(x64[0], x64[1], x64[2], o, lse, x64[3], w.scale)
    check_close("O", f64(got["o"]), o, "fp32")
    check_close("dQ", f64(got["dq"]), dq, "fp32")
    check_close("dK", f64(got["dk"]), dk, "fp32")
    check_close("dV", f64(got["dv"]), dv, "fp32")
    check_close("LSE", np.concatenate([f64(a) for a in lses]), lse, "fp32")


@pytest.mark.parametrize("cu,s_valid,causal", [(None, 200, True), (None, 190, True),
                                               ([0, 50, 51, 200], 200, True),
                                               (None, 190, False)])
def test_fp32_mask_variants(cu, s_valid, causal):
    dev = gpu()
    s, hq, hkv, d = 200, 4, 2, 64
    q, k, v, do = (seeded((s, h, d), 2000 + i, torch.float32) for i, h in enumerate((hq, hkv, hkv, hq)))
    got = run_pair(q, k, v, do, s_valid, cu, causal, dev)
    q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))
    o, lse = oracle.attn_fwd(q64, k64, v64, d ** -0.5, s_valid, cu, causal)
    dq, dk, dv = oracle.attn_bwd(q64, k64, v64, o, lse, do64, d ** -0.5, s_valid, cu, causal)
    for n, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        check_close(n, f64(got[n]), ref, "fp32")


def test_bf16_closed_forms():
    """First row / document-start rows give O = v bit-exactly; K = 0 gives the
    running mean of V and LSE = log(count)."""
    dev = gpu()
    s, hq, hkv, d = 700, 4, 1, 128
    cu = [0, 300, 301, 700]
    q, k, v = (seeded((s, h, d), 3000 + i, torch.bfloat16) for i, h in enumerate((hq, hkv, hkv)))
    got = run_pair(q, k, v, q, s, cu, True, dev, backward=False)
    o = got["o"].cpu()
    for st in cu[:-1]:
        for h in range(hq):
            assert torch.equal(o[st, h].view(torch.int16), v[st, 0].view(torch.int16)), (st, h)
    kz = torch.zeros_like(k)
    got = run_pair(q, kz, v, q, s, None, True, dev, backward=False)
    v64 = f64(v)[:, 0]
    mean = np.cumsum(v64, axis=0) / np.arange(1, s + 1)[:, None]
    check_close("O(K=0)", f64(got["o"]), np.broadcast_to(mean[:, None, :], (s, hq, d)), "bf16")
    np.testing.assert_allclose(f64(got["lse"]), np.broadcast_to(np.log(np.arange(1, s + 1)), (hq, s)),
                               atol=1e-5)


def test_bf16_deterministic():
    dev = gpu()
    s, hq, hkv, d = 1500, 4, 1, 128
    q, k, v, do = (seeded((s, h, d), 4000 + i, torch.bfloat16) for i, h in enumerate((hq, hkv, hkv, hq)))
    a = run_pair(q, k, v, do, s, None, True, dev)
    b = run_pair(q, k, v, do, s, None, True, dev)
    for n in a:
        assert torch.equal(a[n], b[n]), n


# ---------------------------------------------------------------------------
# full-size workloads

def bits(t):
    return t.view(torch.int16).numpy()


def from_bits(a):
    return torch.from_numpy(a).view(torch.bfloat16)


def share_inputs(w, dev):
    """Full-model tensors -> GPU pack -> rank-0 share (GPU), the oracle's own
    pack of the same seeded tensors (CPU, fp64), and a SHA-256 of the
    oracle-packed bf16 bits (which the stored key samples record)."""
    L = usp()
    gpu_in, ref_in, ref_bits = [], [], []
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        x = workloads.tensor(w, t)
        y = L.usp_pad_pack_seq2head(x.to(dev), w.p)
        gpu_in.append(y[0].contiguous())
        del y
        b = oracle.pad_pack_seq2head(bits(x), w.p)[0]
        ref_bits.append(b)
        ref_in.append(from_bits(b).double().numpy())
        del x
    torch.cuda.synchronize()
    return gpu_in, ref_in, input_sha256(ref_bits)


def oracle_by_group(q64, k64, v64, do64, scale, s_valid, cu, causal):
    """Full oracle forward + backward, one KV-head group at a time (the
    groups are independent problems), the groups in parallel threads, each
    with a single-threaded BLAS (nested BLAS threads oversubscribe the host
    many times over)."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits
    hq, hkv = q64.shape[1], k64.shape[1]
    g = hq // hkv

    def one(j):
        qs, ks = slice(g * j, g * (j + 1)), slice(j, j + 1)
        o, lse = oracle.attn_fwd(q64[:, qs], k64[:, ks], v64[:, ks], scale, s_valid, cu, causal)
        dq, dk, dv = oracle.attn_bwd(q64[:, qs], k64[:, ks], v64[:, ks], o, lse, do64[:, qs],
                                     scale, s_valid, cu, causal)
        return o, lse, dq, dk, dv

    with threadpool_limits(1), cf.ThreadPoolExecutor(min(hkv, 16)) as ex:
        parts = list(ex.map(one, range(hkv)))
    cat = [np.concatenate([p[i] for p in parts], axis=1 if i != 1 else 0) for i in range(5)]
    return cat


# Every kernel on its long-sequence path: 64 Q / 16 KV heads at 8192 tokens,
# d = 128. The dK/dV grid then has 1024 (block of 128 keys, KV head) items,
# one row chunk each (the direct-store epilogue of the 120K step), the forward
# 2048 workgroups and dQ 4096 (one pass each, no key splits), so no
# reduction or merge kernel runs. The 8K workload's full model (32 Q / 8 KV)
# runs its dK/dV in two row chunks plus the reduction. Compared element by
# element.
LONG = [
    # name, S, s_valid, cu_seqlens, causal, d, hq, hkv
    ("long_8k_64q16kv", 8192, 8192, None, True, 128, 64, 16),
    ("long_8k_64q16kv_padded", 8192, 8190, None, True, 128, 64, 16),
    ("long_8k_64q16kv_docs", 8192, 8192, [0, 1000, 1001, 5000, 8192], True, 128, 64, 16),
    ("long_8k_32q8kv_two_chunks", 8192, 8192, None, True, 128, 32, 8),
]
SINGLE_PASS = {"attn_fwd_kmajor_v", "attn_fwd_bf16", "attn_bwd_rowdot_bf16",
               "attn_bwd_dkdv_bf16", "attn_bwd_dq_bf16"}


@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_bf16_long_path_full_compare(case):
    name, s, s_valid, cu, causal, d, hq, hkv = case
    L = usp()
    dev = gpu()
    say(f"bf16 {name}: S={s} s_valid={s_valid} hq={hq} hkv={hkv} d={d}")
    assert L.usp_attn_fwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, s_k_valid=s_valid) == 1
    assert L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, s_k_valid=s_valid) == 1
    q, k, v, do = (seeded((s, h, d), 5000 + i, torch.bfloat16)
                   for i, h in enumerate((hq, hkv, hkv, hq)))
    if s_valid < s:
        for t in (q, k, v, do):
            t[s_valid:] = 0
    L.usp_trace_collect()
    L.usp_trace_enable(True)
    try:
        got = run_pair(q, k, v, do, s_valid, cu, causal, dev)
        ran = {e["name"] for e in L.usp_trace_collect()}
    finally:
        L.usp_trace_enable(False)
    # with documents the blocks also run longest first (a plan kernel pair)
    want = SINGLE_PASS | ({"attn_bwd_dkdv_reduce"} if hkv == 8 else set()) | \
        ({"attn_block_order"} if cu is not None else set())
    assert ran == want, ran
    say(f"  oracle, {hkv} groups in parallel")
    o, lse, dq, dk, dv = oracle_by_group(*(f64(t) for t in (q, k, v, do)), d ** -0.5, s_valid, cu,
                                          causal)
    check_close("O", f64(got["o"]), o, "bf16")
    check_close("LSE", f64(got["lse"]), lse, "bf16")
    check_close("dQ", f64(got["dq"]), dq, "bf16")
    check_close("dK", f64(got["dk"]), dk, "bf16")
    check_close("dV", f64(got["dv"]), dv, "bf16")


def test_bf16_document_block_order_only_schedules():
    """With packed documents and one pass per kernel, the forward, dK/dV and dQ
    run their blocks longest first (an order computed on the device from the
    documents). The order only schedules: the outputs equal, bit for bit,
    those of calls whose workspace has no room for it (natural order)."""
    L = usp()
    dev = gpu()
    s, hq, hkv, d = 8192, 64, 16, 128
    cu = [0, 1000, 1001, 5000, 8192]
    say(f"block order: S={s} hq={hq} hkv={hkv} docs={cu}")
    q, k, v, do = (seeded((s, h, d), 5200 + i, torch.bfloat16).to(dev)
                   for i, h in enumerate((hq, hkv, hkv, hq)))
    fw_min = torch.empty(hkv * d * ((s + 127) // 128 * 128) * 2, dtype=torch.uint8, device=dev)
    L.usp_trace_collect()
    L.usp_trace_enable(True)
    try:
        o1, l1 = L.usp_attn_fwd(q, k, v, cu_seqlens=cu)
        g1 = L.usp_attn_bwd(q, k, v, o1, l1, do, cu_seqlens=cu)
        torch.cuda.synchronize()
        ran = {e["name"]: e["launches"] for e in L.usp_trace_collect()}
        o2, l2 = L.usp_attn_fwd(q, k, v, cu_seqlens=cu, workspace=fw_min)
        need = L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16)
        bw_min = torch.empty(need - 1, dtype=torch.uint8, device=dev)  # no room for the orders
        g2 = L.usp_attn_bwd(q, k, v, o1, l1, do, cu_seqlens=cu, workspace=bw_min)
        torch.cuda.synchronize()
        ran2 = {e["name"] for e in L.usp_trace_collect()}
    finally:
        L.usp_trace_enable(False)
    assert ran.get("attn_block_order") == 3, ran  # forward, dK/dV, dQ
    assert "attn_block_order" not in ran2, ran2
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # a contiguous context-parallel rank's rows (global offset, global
    # documents) against every key: also ordered, also bit-identical
    qa = s // 2
    L.usp_trace_collect()
    L.usp_trace_enable(True)
    try:
        o3, l3 = L.usp_attn_fwd_interval(q[qa:], k, v, q_off=qa, cu_seqlens=cu,
                                         out_dtype=torch.bfloat16)
        g3 = L.usp_attn_bwd_interval(q[qa:], k, v, o3, l3, do[qa:], q_off=qa, cu_seqlens=cu)
        torch.cuda.synchronize()
        ran3 = {e["name"]: e["launches"] for e in L.usp_trace_collect()}
        o4, l4 = L.usp_attn_fwd_interval(q[qa:], k, v, q_off=qa, cu_seqlens=cu,
                                         out_dtype=torch.bfloat16, workspace=fw_min)
        nb = L.usp_attn_bwd_interval_workspace_bytes(s - qa, s, hq, hkv, d, L.USP_BF16)
        g4 = L.usp_attn_bwd_interval(q[qa:], k, v, o3, l3, do[qa:], q_off=qa, cu_seqlens=cu,
                                     workspace=torch.empty(nb - 1, dtype=torch.uint8, device=dev))
        torch.cuda.synchronize()
        ran4 = {e["name"] for e in L.usp_trace_collect()}
    finally:
        L.usp_trace_enable(False)
    assert ran3.get("attn_block_order") == 3 and "attn_block_order" not in ran4, (ran3, ran4)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    for a, b in zip(g3, g4):
        assert torch.equal(a, b)
    # the forward's order, read back from its workspace (after the V copy:
    # costs, ranks, then the order), against the CPU replica of the costs
    from tests import kernel_geometry as G
    fw = torch.empty(L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16), dtype=torch.uint8,
                     device=dev)
    L.usp_attn_fwd(q, k, v, cu_seqlens=cu, workspace=fw)
    torch.cuda.synchronize()
    n = -(-s // 64)                            # query blocks of 64 rows (4 heads x 2 x 32)
    part = -(-n * 4 // 256) * 256
    base = hkv * d * ((s + 127) // 128 * 128) * 2
    tab = fw[base:base + 3 * part].cpu().view(torch.int32).numpy()
    m = G.Geom(s_q=s, s_k=s, s_kv=s, cu=cu)
    cost = G.block_costs(m, 0, n, 64, 64)
    np.testing.assert_array_equal(tab[:n], cost)
    np.testing.assert_array_equal(tab[2 * part // 4:2 * part // 4 + n], G.longest_first(cost))
    # the backward's two orders, after its required part (D and LSE*log2(e)
    # rows; no row-chunk partials here): dK/dV key blocks of 128 keys over
    # 64-row tiles, then dQ query blocks of 32 rows over 32-key tiles
    bw = torch.empty(L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16), dtype=torch.uint8,
                     device=dev)
    L.usp_attn_bwd(q, k, v, o1, l1, do, cu_seqlens=cu, workspace=bw)
    torch.cuda.synchronize()
    req = 2 * (-(-hq * ((s + 127) // 128 * 128) * 4 // 256) * 256)
    for kind, nb, block, tile in ((1, -(-s // 128), 128, 64), (0, -(-s // 32), 32, 32)):
        part = -(-nb * 4 // 256) * 256
        tab = bw[req:req + 3 * part].cpu().view(torch.int32).numpy()
        cost = G.block_costs(m, kind, nb, block, tile)
        np.testing.assert_array_equal(tab[:nb], cost)
        np.testing.assert_array_equal(tab[2 * part // 4:2 * part // 4 + nb], G.longest_first(cost))
        req += 3 * part


def key_fixture(name):
    """Stored oracle dK / dV on the full-size key sample (written by
    tests/golden/make_full_size_keys.py from the oracle alone)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_size_keys",
                        f"{name}.npz")
    with np.load(path, allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def input_sha256(arrays_bits):
    import hashlib
    h = hashlib.sha256()
    for a in arrays_bits:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", ["s8k", "s32k", "s120k", "s120k_pad", "thd131k"])
def test_workload(name):
    L = usp()
    dev = gpu()
    w = workloads.WORKLOADS[name]
    cu = workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if w.thd else None
    say(f"{name}: generating + packing S={w.s} (s_pad={w.s_pad}) hq={w.hq} hkv={w.hkv}")
    (q, k, v, do), (q64, k64, v64, do64), sha = share_inputs(w, dev)
    say(f"{name}: forward")
    o, lse = L.usp_attn_fwd(q, k, v, s_valid=w.s, cu_seqlens=cu)
    torch.cuda.synchronize()
    if w.backward:
        say(f"{name}: backward")
        dq, dk, dv = L.usp_attn_bwd(q, k, v, o, lse, do, s_valid=w.s, cu_seqlens=cu)
        torch.cuda.synchronize()
    scale = w.scale
    rows = workloads.row_sample(w)
    say(f"{name}: oracle on {len(rows)} sampled rows")
    o_ref, lse_ref = oracle.attn_fwd_rows(q64, k64, v64, rows, scale, w.s, cu)
    check_close("O[rows]", f64(o)[rows], o_ref, "bf16")
    check_close("LSE[rows]", f64(lse)[:, rows], lse_ref, "bf16")
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(lse)).all()
    if not w.backward:
        return
    dq_ref = oracle.attn_bwd_rows(q64, k64, v64, do64, rows, scale, w.s, cu, lse=lse_ref)
    check_close("dQ[rows]", f64(dq)[rows], dq_ref, "bf16")
    # dK / dV on the same sample as keys, against the stored oracle values
    fx = key_fixture(name)
    assert str(fx["inputs_sha256"]) == sha, "stored key sample was made from other inputs"
    keys = fx["keys"]
    np.testing.assert_array_equal(keys, rows)
    dk64, dv64, do_all = f64(dk), f64(dv), do64
    say(f"{name}: dK/dV on {len(keys)} sampled keys")
    check_close("dK[keys]", dk64[keys], fx["dk"].astype(np.float64), "bf16",
                bound=rounding_bound(fx["dk"], fx["adk"], 2))
    check_close("dV[keys]", dv64[keys], fx["dv"].astype(np.float64), "bf16",
                bound=rounding_bound(fx["dv"], fx["adv"], 1))
    for a in (f64(dq), dk64, dv64):
        assert np.isfinite(a).all()
    # identities over the full outputs, per document: sum_j dK_j = 0 and
    # sum_j dV_j = sum over the group's heads and the document's rows of dO
    g = w.hq // w.hkv
    spans = [(0, w.s_pad)] if cu is None else list(zip(cu[:-1], cu[1:]))
    for a, b in spans:
        sk = dk64[a:b].sum(axis=0)
        assert np.abs(sk).max() <= 1e-3 * np.abs(dk64[a:b]).sum(axis=0).max() + 1e-3, (a, b)
        sv = dv64[a:b].sum(axis=0)
        rhs = do_all[a:b].reshape(b - a, w.hkv, g, -1).sum(axis=(0, 2))
        err = np.abs(sv - rhs).max()
        say(f"  identity span [{a},{b}): |sum dK| {np.abs(sk).max():.3e}  |sum dV - sum dO| {err:.3e}")
        assert err <= 1e-3 * np.abs(dv64[a:b]).sum(axis=0).max() + 1e-3, (a, b, err)
    if w.s < w.s_pad:
        assert (dk64[w.s:] == 0).all() and (dv64[w.s:] == 0).all()


def test_a_single_host_tensor_is_refused():
    """GPU inputs with one host tensor among the outputs or the workspace: the
    binding refuses the call before the library sees a host pointer."""
    import ulysses_sequence_parallelism_amd as L
    dev = gpu()
    q = torch.zeros((128, 4, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((128, 1, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    with pytest.raises(ValueError, match="must be on a GPU"):
        L.usp_attn_fwd(q, k, v, out=torch.zeros((128, 4, 128), dtype=torch.bfloat16))
    ws = torch.empty(L.usp_attn_fwd_workspace_bytes(128, 4, 1, 128, L.USP_BF16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="must be on a GPU"):
        L.usp_attn_fwd(q, k, v, workspace=ws)
    o, lse = L.usp_attn_fwd(q, k, v)  # the same call on the GPU goes through
    torch.cuda.synchronize()
    assert o.is_cuda and lse.is_cuda


# The forward runs two wave groups half a tile apart, with a barrier between
# its softmax and matrix phases, a tile loop unrolled by three, and an extra
# barrier for each group outside the loop. Every tile count modulo three, and
# key splits that leave a workgroup few or no tiles, go through different
# parts of that schedule.
# Bidirectional S = 64 n gives every workgroup exactly n key tiles in one pass;
# from about 1,000 rows the recommended workspace lets the call split (2 to 7
# splits here), and causal splits of the early query blocks get no tiles.
TILE_COUNTS = ([(64 * n, False, False) for n in range(1, 10)]
               + [(64 * n + 17, True, False) for n in (1, 2, 3, 5)]
               + [(1024, False, True), (1500, False, True), (3000, True, True), (4096, True, True)])


@pytest.mark.parametrize("s,causal,splits_expected", TILE_COUNTS,
                         ids=[f"S{s}_{'causal' if c else 'bidir'}" for s, c, _ in TILE_COUNTS])
def test_bf16_forward_tile_counts_one_pass_and_split(s, causal, splits_expected):
    L = usp()
    dev = gpu()
    hq, hkv, d = 4, 1, 128
    q, k, v = (seeded((s, h, d), 3000 + s + i, torch.bfloat16) for i, h in enumerate((hq, hkv, hkv)))
    q64, k64, v64 = (f64(t) for t in (q, k, v))
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, d ** -0.5, s, None, causal)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    minimum = hkv * d * (-(-s // 128) * 128) * 2
    full = L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16)
    splits = []
    for ws_bytes in (minimum, full):
        z = L.usp_attn_fwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, causal=causal,
                                      workspace_bytes=ws_bytes)
        splits.append(z)
        say(f"S={s} causal={causal} workspace={ws_bytes} key splits={z}")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        o, lse = L.usp_attn_fwd(qd, kd, vd, causal=causal, workspace=ws)
        torch.cuda.synchronize()
        check_close("O", f64(o), o_ref, "bf16")
        check_close("LSE", f64(lse), lse_ref, "bf16")
    assert splits[0] == 1
    assert (splits[1] > 1) == splits_expected, splits
