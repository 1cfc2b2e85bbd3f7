"""GPU parity of usp_attn_fwd / usp_attn_bwd against the fp64 oracle.

Small problems (several tiles plus a ragged tail) are compared element by
element over every output; the full-size workloads are compared on sampled
query rows (O, LSE, dQ), on key rows near the end of the sequence or of each
document (dK, dV: few query rows see them, so the oracle computes them
exactly), and through identities that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import check_close, f64, gpu, say

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
    ("bidirectional_docs", 600, 600, 4, 2, [0, 250, 600], False),
    # shorter than one 32-row block: every tile is a ragged tail
    ("tiny_1", 1, 1, 4, 1, None, True),
    ("tiny_17", 17, 17, 4, 1, None, True),
    ("tiny_bidir_33", 33, 30, 4, 2, None, False),
    # 8 query heads per KV head: two head chunks per KV head
    ("gqa8", 300, 300, 8, 1, None, True),
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
    """Full-model tensors -> GPU pack -> rank-0 share (GPU), and the oracle's
    own pack of the same seeded tensors (CPU, fp64)."""
    L = usp()
    gpu_in, ref_in = [], []
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        x = workloads.tensor(w, t)
        y = L.usp_pad_pack_seq2head(x.to(dev), w.p)
        gpu_in.append(y[0].contiguous())
        del y
        ref_in.append(from_bits(oracle.pad_pack_seq2head(bits(x), w.p)[0]).double().numpy())
        del x
    torch.cuda.synchronize()
    return gpu_in, ref_in


def tail_keys(w, cu):
    ends = [w.s_pad] if cu is None else list(cu[1:])
    keys = set()
    for e in ends:
        keys.update(range(max(0, e - 24), e))
    return np.array(sorted(keys), dtype=np.int64)


@pytest.mark.parametrize("name", ["s8k", "s32k", "s120k", "s120k_pad", "thd131k"])
def test_workload(name):
    L = usp()
    dev = gpu()
    w = workloads.WORKLOADS[name]
    cu = workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if w.thd else None
    say(f"{name}: generating + packing S={w.s} (s_pad={w.s_pad}) hq={w.hq} hkv={w.hkv}")
    (q, k, v, do), (q64, k64, v64, do64) = share_inputs(w, dev)
    say(f"{name}: forward")
    o, lse = L.usp_attn_fwd(q, k, v, s_valid=w.s, cu_seqlens=cu)
    torch.cuda.synchronize()
    if w.backward:
        say(f"{name}: backward")
        dq, dk, dv = L.usp_attn_bwd(q, k, v, o, lse, do, s_valid=w.s, cu_seqlens=cu)
        torch.cuda.synchronize()
    scale = w.scale
    slice_edges = [r * (w.s_pad // w.p) for r in range(1, w.p)]
    rows = workloads.row_sample(w, n_uniform=160, edge=16,
                                boundaries=slice_edges + (cu[1:-1] if cu else []))
    say(f"{name}: oracle on {len(rows)} sampled rows")
    o_ref, lse_ref = oracle.attn_fwd_rows(q64, k64, v64, rows, scale, w.s, cu)
    check_close("O[rows]", f64(o)[rows], o_ref, "bf16")
    check_close("LSE[rows]", f64(lse)[:, rows], lse_ref, "bf16")
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(lse)).all()
    if not w.backward:
        return
    dq_ref = oracle.attn_bwd_rows(q64, k64, v64, do64, rows, scale, w.s, cu)
    check_close("dQ[rows]", f64(dq)[rows], dq_ref, "bf16")
    keys = tail_keys(w, cu)
    say(f"{name}: oracle dK/dV on {len(keys)} tail keys")
    dk_ref, dv_ref = oracle.attn_bwd_keys(q64, k64, v64, do64, keys, scale, w.s, cu)
    dk64, dv64, do_all = f64(dk), f64(dv), do64
    check_close("dK[keys]", dk64[keys], dk_ref, "bf16")
    check_close("dV[keys]", dv64[keys], dv_ref, "bf16")
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
