"""GPU parity of the interval entry points (usp_attn_fwd_interval,
usp_attn_merge, usp_attn_bwd_interval) against the fp64 oracle.

Ring / USP attention splits the key axis into blocks (one per ring step) and
merges the partial results; contiguous context parallelism splits the query
axis, each rank's rows carrying their global offset. Both are checked
element by element on small problems (every partial against
oracle.attn_fwd_partial / attn_bwd_partial, the merged result and the summed
gradients against full attention), on the edge cases (blocks entirely in the
future, merge identities, padded last block), and on sampled rows of a
32K-token share split four ways."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import check_close, f64, gpu, rounding_bound, say
from tests.test_gpu_attention import bits, input_sha256, key_fixture

pytestmark = pytest.mark.gpu


def usp():
    import ulysses_sequence_parallelism_amd as m
    return m


def seeded(shape, seed, dtype):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))
    return x.to(dtype)


def check_partial(name, o, lse, o_ref, lse_ref, dtype):
    """Partial results: rows without an allowed key must be exactly O = 0 and
    LSE = -inf on both sides; the rest meet the dtype's bar."""
    o, lse = f64(o), f64(lse)
    empty = np.isneginf(lse_ref)
    assert (np.isneginf(lse) == empty).all(), f"{name}: empty-row pattern differs"
    assert (o.transpose(1, 0, 2)[empty] == 0).all(), f"{name}: empty rows not zero"
    live = ~empty
    if live.any():
        check_close(f"{name} O", o.transpose(1, 0, 2)[live], o_ref.transpose(1, 0, 2)[live],
                    dtype, bf16_out=False)
        check_close(f"{name} LSE", lse[live], lse_ref[live], dtype)


def edges_of(e):
    return list(zip(e[:-1], e[1:]))


CASES = [
    # name, S, s_valid, hq, hkv, query edges, key edges, cu_seqlens, causal
    ("ring4", 1024, 1024, 8, 2, [0, 1024], [0, 256, 512, 768, 1024], None, True),
    ("ring_ragged", 1000, 1000, 4, 1, [0, 1000], [0, 300, 301, 700, 1000], None, True),
    ("usp_grid", 900, 900, 4, 2, [0, 333, 900], [0, 100, 450, 900], None, True),
    ("ring_docs", 1500, 1500, 4, 1, [0, 1500], [0, 500, 1000, 1500],
     [0, 200, 777, 1300, 1500], True),
    ("cp_docs", 1200, 1200, 8, 2, [0, 300, 701, 1200], [0, 1200], [0, 333, 900, 1200], True),
    ("bidir_padded", 900, 890, 4, 2, [0, 900], [0, 300, 600, 900], None, False),
    ("bidir_grid_docs", 640, 640, 4, 1, [0, 200, 640], [0, 320, 640], [0, 250, 640], False),
    # one-row query interval, one-key and two-key key intervals
    ("single_rows", 70, 70, 4, 1, [0, 1, 70], [0, 1, 3, 70], None, True),
    ("single_rows_bidir", 70, 66, 4, 2, [0, 1, 69, 70], [0, 1, 3, 70], None, False),
    # head dim 64
    ("d64_usp_grid", 900, 900, 4, 2, [0, 333, 900], [0, 100, 450, 900], None, True, 64),
    ("d64_cp_docs", 1200, 1200, 8, 2, [0, 300, 701, 1200], [0, 1200], [0, 333, 900, 1200], True,
     64),
    ("d64_bidir_padded", 900, 890, 4, 1, [0, 900], [0, 300, 600, 900], None, False, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_interval_split_forward_backward(case):
    """Split queries and keys into intervals, run every (query, key) pair,
    merge forward partials over the key intervals, accumulate dQ over the key
    intervals and dK / dV over the query intervals; compare partials and
    totals with the oracle."""
    name, s, s_valid, hq, hkv, qe, ke, cu, causal = case[:9]
    d = case[9] if len(case) > 9 else 128
    L = usp()
    dev = gpu()
    scale = d ** -0.5
    say(f"interval {name}: S={s} hq={hq} hkv={hkv} d={d} q={qe} k={ke} causal={causal}")
    q, k, v, do = (seeded((s, h, d), 5000 + i, torch.bfloat16)
                   for i, h in enumerate((hq, hkv, hkv, hq)))
    if s_valid < s:
        for t in (q, k, v, do):
            t[s_valid:] = 0
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))

    o_fin = torch.empty((s, hq, d), dtype=torch.bfloat16, device=dev)
    lse_rows = []
    for qa, qb in edges_of(qe):
        acc_o = acc_l = None
        for r, (ka, kb) in enumerate(edges_of(ke)):
            skv = max(0, min(kb, s_valid) - ka)
            o_p, l_p = L.usp_attn_fwd_interval(qd[qa:qb], kd[ka:kb], vd[ka:kb], q_off=qa,
                                               k_off=ka, s_k_valid=skv, cu_seqlens=cu,
                                               causal=causal)
            torch.cuda.synchronize()
            o_r, l_r = oracle.attn_fwd_partial(q64[qa:qb], k64[ka:kb], v64[ka:kb], scale, qa, ka,
                                               skv, cu, causal)
            check_partial(f"part q[{qa},{qb}) k[{ka},{kb})", o_p, l_p, o_r, l_r, "bf16")
            if acc_o is None:
                acc_o, acc_l = o_p, l_p
            else:
                L.usp_attn_merge(acc_o, acc_l, o_p, l_p, out=acc_o, lse=acc_l)  # in place
        # final rows in bf16 (a second merge with an empty partial converts)
        empty_o = torch.zeros_like(acc_o)
        empty_l = torch.full_like(acc_l, -float("inf"))
        _, l_fin = L.usp_attn_merge(acc_o, acc_l, empty_o, empty_l, out=o_fin[qa:qb])
        lse_rows.append(l_fin)
    lse_fin = torch.cat(lse_rows, dim=1)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, s_valid, cu, causal)
    check_close("merged O", f64(o_fin), o_ref, "bf16")
    check_close("merged LSE", f64(lse_fin), lse_ref, "bf16")

    # backward over the same grid, fp32 accumulation in place
    dq = torch.zeros((s, hq, d), dtype=torch.float32, device=dev)
    dk = torch.zeros((s, hkv, d), dtype=torch.float32, device=dev)
    dv = torch.zeros((s, hkv, d), dtype=torch.float32, device=dev)
    checked_pair = False
    for qa, qb in edges_of(qe):
        for ka, kb in edges_of(ke):
            skv = max(0, min(kb, s_valid) - ka)
            args = (qd[qa:qb], kd[ka:kb], vd[ka:kb], o_fin[qa:qb], lse_fin[:, qa:qb].contiguous(),
                    dod[qa:qb])
            if not checked_pair:
                # one pair on its own, written (not accumulated), against the oracle
                a, b, c = L.usp_attn_bwd_interval(*args, q_off=qa, k_off=ka, s_k_valid=skv,
                                                  cu_seqlens=cu, causal=causal)
                torch.cuda.synchronize()
                ra, rb, rc = oracle.attn_bwd_partial(
                    q64[qa:qb], k64[ka:kb], v64[ka:kb], f64(o_fin[qa:qb]), f64(lse_fin[:, qa:qb]),
                    do64[qa:qb], scale, qa, ka, skv, cu, causal)
                check_close("pair dQ", f64(a), ra, "bf16", bf16_out=False)
                check_close("pair dK", f64(b), rb, "bf16", bf16_out=False)
                check_close("pair dV", f64(c), rc, "bf16", bf16_out=False)
                checked_pair = True
            L.usp_attn_bwd_interval(*args, q_off=qa, k_off=ka, s_k_valid=skv, cu_seqlens=cu,
                                    causal=causal, accumulate=True, dq=dq[qa:qb], dk=dk[ka:kb],
                                    dv=dv[ka:kb])
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attn_bwd(q64, k64, v64, o_ref, lse_ref, do64, scale, s_valid, cu,
                                    causal)
    check_close("summed dQ", f64(dq), rdq, "bf16", bf16_out=False)
    check_close("summed dK", f64(dk), rdk, "bf16", bf16_out=False)
    check_close("summed dV", f64(dv), rdv, "bf16", bf16_out=False)


def test_bf16_contiguous_cp_rows_equal_full_attention_rows():
    """A contiguous context-parallel rank: its query rows (global offset)
    against the whole key sequence, bf16 O written directly, equal the same
    rows of the full-sequence call; its bf16 dQ equals the same rows of the
    full-sequence dQ (both against the oracle)."""
    L = usp()
    dev = gpu()
    s, hq, hkv, d = 1100, 8, 2, 128
    cu = [0, 400, 401, 1100]
    q, k, v, do = (seeded((s, h, d), 6000 + i, torch.bfloat16)
                   for i, h in enumerate((hq, hkv, hkv, hq)))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))
    scale = d ** -0.5
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, None, cu, True)
    dq_ref, _, _ = oracle.attn_bwd(q64, k64, v64, o_ref, lse_ref, do64, scale, None, cu, True)
    for qa, qb in ((0, 275), (275, 550), (550, 825), (825, 1100)):
        o, lse = L.usp_attn_fwd_interval(qd[qa:qb], kd, vd, q_off=qa, k_off=0, cu_seqlens=cu,
                                         out_dtype=torch.bfloat16)
        dq, _, _ = L.usp_attn_bwd_interval(qd[qa:qb], kd, vd, o, lse, dod[qa:qb], q_off=qa,
                                           cu_seqlens=cu, grad_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        check_close(f"O rows [{qa},{qb})", f64(o), o_ref[qa:qb], "bf16")
        check_close(f"LSE rows [{qa},{qb})", f64(lse), lse_ref[:, qa:qb], "bf16")
        check_close(f"dQ rows [{qa},{qb})", f64(dq), dq_ref[qa:qb], "bf16")


def test_bf16_future_key_block_is_empty():
    """Keys entirely after every query row (causal): every row is empty (O = 0,
    LSE = -inf), and the backward adds exactly nothing."""
    L = usp()
    dev = gpu()
    hq, hkv, d = 4, 1, 128
    q = seeded((200, hq, d), 7000, torch.bfloat16).to(dev)
    k, v = (seeded((300, hkv, d), 7001 + i, torch.bfloat16).to(dev) for i in range(2))
    o, lse = L.usp_attn_fwd_interval(q, k, v, q_off=0, k_off=200)
    torch.cuda.synchronize()
    assert torch.isneginf(lse).all() and (o == 0).all()
    # partly visible block: rows >= 200 - q_off see a prefix
    o2, lse2 = L.usp_attn_fwd_interval(q, k, v, q_off=150, k_off=200)
    torch.cuda.synchronize()
    l2 = f64(lse2)
    assert np.isneginf(l2[:, :50]).all() and np.isfinite(l2[:, 50:]).all()
    # row 50 (global 200) sees key 0 only: O = v_0 exactly
    assert torch.equal(o2[50].to(torch.bfloat16).cpu().view(torch.int16),
                       v[0, 0].cpu().view(torch.int16).expand(hq, d))
    do = seeded((200, hq, d), 7003, torch.bfloat16).to(dev)
    o_fin = seeded((200, hq, d), 7004, torch.bfloat16).to(dev)
    lse_fin = torch.randn((hq, 200), device=dev)
    dq = torch.full((200, hq, d), 3.0, device=dev)
    dk = torch.full((300, hkv, d), -2.0, device=dev)
    dv = torch.full((300, hkv, d), 5.0, device=dev)
    L.usp_attn_bwd_interval(q, k, v, o_fin, lse_fin, do, q_off=0, k_off=200, accumulate=True,
                            dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dq == 3.0).all() and (dk == -2.0).all() and (dv == 5.0).all()


def test_merge_identities_and_oracle():
    L = usp()
    dev = gpu()
    s, hq = 333, 6
    for d in (64, 128):
        o_a = torch.randn((s, hq, d), device=dev)
        o_b = torch.randn((s, hq, d), device=dev)
        l_a = torch.randn((hq, s), device=dev) * 30
        l_b = torch.randn((hq, s), device=dev) * 30
        l_a[0, :7] = -float("inf")                    # a empty on some rows
        l_b[1, 3:9] = -float("inf")                   # b empty on others
        l_a[2, 10:12] = l_b[2, 10:12] = -float("inf")  # both empty
        o_a[:7, 0] = 0
        o_b[3:9, 1] = 0
        o_a[10:12, 2] = o_b[10:12, 2] = 0
        o, lse = L.usp_attn_merge(o_a, l_a, o_b, l_b)
        torch.cuda.synchronize()
        ro, rl = oracle.lse_merge([(f64(o_a), f64(l_a)), (f64(o_b), f64(l_b))])
        got_l = f64(lse)
        assert (np.isneginf(got_l) == np.isneginf(rl)).all()
        fin = np.isfinite(rl)
        np.testing.assert_allclose(got_l[fin], rl[fin], rtol=1e-6, atol=1e-5)
        np.testing.assert_allclose(f64(o), ro, rtol=1e-5, atol=1e-5)
        # identity: merging with an empty partial returns the other one bit for bit
        empty_o = torch.zeros_like(o_a)
        empty_l = torch.full_like(l_a, -float("inf"))
        o2, l2 = L.usp_attn_merge(o_a, l_a, empty_o, empty_l)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_a) and torch.equal(l2, l_a)
        # merging a partial with itself: O unchanged, LSE + log 2
        o3, l3 = L.usp_attn_merge(o_b, l_b, o_b, l_b)
        torch.cuda.synchronize()
        assert torch.equal(o3, o_b)
        fin = torch.isfinite(l_b)
        torch.testing.assert_close(l3[fin], l_b[fin] + float(np.log(2.0)), rtol=1e-6, atol=1e-5)
        # bf16 output rounds the fp32 result once (round to nearest even)
        o4, _ = L.usp_attn_merge(o_a, l_a, o_b, l_b, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o4, o.to(torch.bfloat16))


@pytest.mark.parametrize("causal", [True, False])
def test_fp32_interval_split(causal):
    """fp32 path (d = 64): ring split into three key blocks with a padded last
    block, merge, accumulated backward; 1e-4 bar."""
    L = usp()
    dev = gpu()
    s, s_valid, hq, hkv, d = 300, 293, 4, 2, 64
    scale = d ** -0.5
    q, k, v, do = (seeded((s, h, d), 8000 + i, torch.float32) for i, h in enumerate((hq, hkv, hkv, hq)))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))
    ke = [0, 90, 91, 300]
    acc_o = acc_l = None
    for ka, kb in edges_of(ke):
        skv = max(0, min(kb, s_valid) - ka)
        o_p, l_p = L.usp_attn_fwd_interval(qd, kd[ka:kb], vd[ka:kb], k_off=ka, s_k_valid=skv,
                                           causal=causal)
        torch.cuda.synchronize()
        o_r, l_r = oracle.attn_fwd_partial(q64, k64[ka:kb], v64[ka:kb], scale, 0, ka, skv, None,
                                           causal)
        check_partial(f"fp32 part k[{ka},{kb})", o_p, l_p, o_r, l_r, "fp32")
        if acc_o is None:
            acc_o, acc_l = o_p, l_p
        else:
            L.usp_attn_merge(acc_o, acc_l, o_p, l_p, out=acc_o, lse=acc_l)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q64, k64, v64, scale, s_valid, None, causal)
    check_close("fp32 merged O", f64(acc_o), o_ref, "fp32")
    check_close("fp32 merged LSE", f64(acc_l), lse_ref, "fp32")
    dq = torch.zeros_like(qd)
    dk = torch.zeros_like(kd)
    dv = torch.zeros_like(vd)
    for ka, kb in edges_of(ke):
        skv = max(0, min(kb, s_valid) - ka)
        L.usp_attn_bwd_interval(qd, kd[ka:kb], vd[ka:kb], acc_o, acc_l, dod, k_off=ka,
                                s_k_valid=skv, causal=causal, accumulate=True, dq=dq,
                                dk=dk[ka:kb], dv=dv[ka:kb])
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attn_bwd(q64, k64, v64, o_ref, lse_ref, do64, scale, s_valid, None,
                                    causal)
    check_close("fp32 summed dQ", f64(dq), rdq, "fp32")
    check_close("fp32 summed dK", f64(dk), rdk, "fp32")
    check_close("fp32 summed dV", f64(dv), rdv, "fp32")


def test_bf16_ring4_on_32k_share_sampled_rows():
    """The 32K-token rank share (4 query heads / 1 KV head, d = 128) as a ring
    of four key blocks: merged O / LSE on sampled rows against the oracle, and
    against the single-call forward everywhere (bf16 rounding of O apart)."""
    L = usp()
    dev = gpu()
    w = workloads.WORKLOADS["s32k"]
    say(f"ring4 on {w.name}: S={w.s} hq={w.hq} hkv={w.hkv}")
    x = {}
    for t in (workloads.Q, workloads.K, workloads.V):
        full = workloads.tensor(w, t)
        x[t] = L.usp_pad_pack_seq2head(full.to(dev), w.p)[0].contiguous()
        del full
    q, k, v = x[workloads.Q], x[workloads.K], x[workloads.V]
    s = q.shape[0]
    blk = [0, s // 4, s // 2, 3 * s // 4, s]
    acc_o = acc_l = None
    for ka, kb in edges_of(blk):
        skv = max(0, min(kb, w.s) - ka)
        o_p, l_p = L.usp_attn_fwd_interval(q, k[ka:kb], v[ka:kb], k_off=ka, s_k_valid=skv,
                                           softmax_scale=w.scale)
        if acc_o is None:
            acc_o, acc_l = o_p, l_p
        else:
            L.usp_attn_merge(acc_o, acc_l, o_p, l_p, out=acc_o, lse=acc_l)
    o_full, lse_full = L.usp_attn_fwd(q, k, v, s_valid=w.s, softmax_scale=w.scale)
    torch.cuda.synchronize()
    rows = workloads.row_sample(w, n_uniform=96, edge=8, boundaries=blk[1:-1])
    q64, k64, v64 = (f64(t) for t in (q, k, v))
    o_ref, lse_ref = oracle.attn_fwd_rows(q64, k64, v64, rows, w.scale, w.s, None)
    check_close("ring O[rows]", f64(acc_o)[rows], o_ref, "bf16", bf16_out=False)
    check_close("ring LSE[rows]", f64(acc_l)[:, rows], lse_ref, "bf16")
    # everywhere: the merged fp32 O and the single call's bf16 O differ by the
    # bf16 rounding of O plus accumulation-order effects
    diff = (acc_o - o_full.float()).abs()
    say(f"  ring vs single call: max {diff.max().item():.3e} mean {diff.mean().item():.3e}")
    assert diff.max().item() <= 2e-2 and diff.mean().item() <= 2e-3
    torch.testing.assert_close(acc_l, lse_full, rtol=0, atol=2e-2)


def test_bf16_usp_ulysses2_ring4_last_rank_120k():
    """One GPU's share of USP on 8 GPUs as Ulysses 2 x Ring 4 at S = 120000:
    the heads of Ulysses group 0 (16 Q / 4 KV), the last ring rank's 30000
    query rows against the four key blocks in ring order. Merged O / LSE and
    the accumulated dQ on sampled rows of the rank, and dK / dV on keys
    sampled over the whole sequence (this rank's rows' contributions, stored
    by tests/golden/make_full_size_keys.py), against the oracle."""
    L = usp()
    dev = gpu()
    w = workloads.WORKLOADS["s120k"]
    u, r = 2, 4
    hq, hkv = w.hq_full // u, w.hkv_full // u
    s = w.s
    say(f"USP U{u}xR{r} at S={s}: {hq} Q / {hkv} KV heads")
    x = {}
    for t in (workloads.Q, workloads.K, workloads.V, workloads.DO):
        full = workloads.tensor(w, t)
        x[t] = full[:, : full.shape[1] // u].contiguous()
        del full
    q, k, v, do = (x[t].to(dev) for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    blk = s // r
    qa, qb = (r - 1) * blk, s
    acc_o = acc_l = None
    for j in [r - 1] + list(range(r - 2, -1, -1)):
        ka, kb = j * blk, (j + 1) * blk
        o_p, l_p = L.usp_attn_fwd_interval(q[qa:qb], k[ka:kb], v[ka:kb], q_off=qa, k_off=ka,
                                           softmax_scale=w.scale)
        if acc_o is None:
            acc_o, acc_l = o_p, l_p
        else:
            L.usp_attn_merge(acc_o, acc_l, o_p, l_p, out=acc_o, lse=acc_l)
    o_fin = acc_o.to(torch.bfloat16)
    dq = torch.zeros((blk, hq, w.d), dtype=torch.float32, device=dev)
    dk = torch.zeros((s, hkv, w.d), dtype=torch.float32, device=dev)
    dv = torch.zeros((s, hkv, w.d), dtype=torch.float32, device=dev)
    for j in range(r):
        ka, kb = j * blk, (j + 1) * blk
        L.usp_attn_bwd_interval(q[qa:qb], k[ka:kb], v[ka:kb], o_fin, acc_l, do[qa:qb], q_off=qa,
                                k_off=ka, softmax_scale=w.scale, accumulate=True, dq=dq,
                                dk=dk[ka:kb], dv=dv[ka:kb])
    torch.cuda.synchronize()
    # rows: the rank's first and last 64 and 256 seeded uniform rows (each
    # costs the oracle a full 16-head row); keys: the full-size sample over the
    # whole sequence, against stored oracle values of this rank's rows'
    # contributions
    rows = workloads.index_sample(s, [w.cfg, 7, 9], 256, 64, [], lo=qa)
    q64, k64, v64, do64 = (f64(x[t]) for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    say(f"  oracle on {len(rows)} rows")
    o_ref, lse_ref = oracle.attn_fwd_rows(q64, k64, v64, rows, w.scale)
    check_close("USP O[rows]", f64(acc_o)[rows - qa], o_ref, "bf16", bf16_out=False)
    check_close("USP LSE[rows]", f64(acc_l)[:, rows - qa], lse_ref, "bf16")
    dq_ref = oracle.attn_bwd_rows(q64, k64, v64, do64, rows, w.scale, lse=lse_ref)
    check_close("USP dQ[rows]", f64(dq)[rows - qa], dq_ref, "bf16", bf16_out=False)
    fx = key_fixture("usp_u2r4_120k")
    assert str(fx["inputs_sha256"]) == input_sha256([bits(x[t]) for t in (
        workloads.Q, workloads.K, workloads.V, workloads.DO)]), "stored keys made from other inputs"
    assert int(fx["q_lo"]) == qa and int(fx["q_hi"]) == qb
    keys = fx["keys"]
    say(f"  dK/dV on {len(keys)} sampled keys")
    check_close("USP dK[keys]", f64(dk)[keys], fx["dk"].astype(np.float64), "bf16", bf16_out=False,
                bound=rounding_bound(fx["dk"], fx["adk"], 2, bf16_output=False))
    check_close("USP dV[keys]", f64(dv)[keys], fx["dv"].astype(np.float64), "bf16", bf16_out=False,
                bound=rounding_bound(fx["dv"], fx["adv"], 1, bf16_output=False))
    # keys of the first block are seen by every one of this rank's rows: finite, nonzero
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all() and dk[:blk].abs().sum() > 0
