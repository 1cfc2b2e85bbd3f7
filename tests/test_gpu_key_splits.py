"""GPU parity of the key splits of the bf16 forward and dQ kernels.

On short sequences both query-stationary kernels cut each query block's key
tiles into several ranges run by separate workgroups. The forward writes fp32
partial O / LSE and a merge kernel combines them exactly. dQ writes fp32
partial sums and a reduction adds them in split order. Every case here is one
the planner splits for both kernels (asserted through usp_attn_fwd_num_splits
and usp_attn_bwd_num_splits). Each runs twice on the same inputs: with the
workspaces the queries return (split) and with the required parts alone (one
pass). Both are compared with the fp64 oracle, element by element, or on
sampled rows at 8K."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, f64, gpu, say
from tests.test_capi_cpu import dq_room

pytestmark = pytest.mark.gpu


def usp():
    import ulysses_sequence_parallelism_amd as m
    return m


def seeded(shape, seed, dtype=torch.bfloat16):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))
    return x.to(dtype)


def vcopy_bytes(s_k, hkv, d):
    return hkv * d * ((s_k + 127) // 128 * 128) * 2


def bwd_workspaces(L, s_q, s_k, hq, hkv, d, dev):
    """(workspace the query returns, its required part alone) for the backward."""
    full = L.usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, L.USP_BF16)
    req = full - dq_room(s_q, hq, hkv, d, s_k)
    return (torch.empty(full, dtype=torch.uint8, device=dev),
            torch.empty(req, dtype=torch.uint8, device=dev))


FULL = [
    # name, S, s_valid, hq, hkv, cu_seqlens, causal, d
    ("causal_1000", 1000, 1000, 4, 1, None, True, 128),
    ("padded_bidir", 1500, 1490, 4, 1, None, False, 128),
    ("docs", 2100, 2100, 4, 1, [0, 100, 101, 1000, 1377, 2100], True, 128),
    ("gqa2_d64", 2048, 2048, 4, 2, None, True, 64),
    ("docs_16q4kv", 2048, 2048, 16, 4, [0, 700, 1300, 2048], True, 128),
    ("gqa8_ragged", 3001, 3001, 8, 1, None, True, 128),
    ("mha_d64_bidir", 1200, 1200, 2, 2, None, False, 64),
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_split_forward_full_compare(case):
    name, s, s_valid, hq, hkv, cu, causal, d = case
    L = usp()
    dev = gpu()
    n = L.usp_attn_fwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, causal=causal, s_k_valid=s_valid)
    nb = L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, causal=causal, s_k_valid=s_valid)
    say(f"splits {name}: S={s} s_valid={s_valid} hq={hq} hkv={hkv} d={d} causal={causal} "
        f"fwd splits={n} dq splits={nb}")
    assert n > 1 and nb > 1
    q, k, v, do = (seeded((s, h, d), 2000 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    if s_valid < s:
        for t in (q, k, v, do):
            t[s_valid:] = 0
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o_s, lse_s = L.usp_attn_fwd(qd, kd, vd, s_valid=s_valid, cu_seqlens=cu, causal=causal)
    ws1 = torch.empty(vcopy_bytes(s, hkv, d), dtype=torch.uint8, device=dev)
    o_1, lse_1 = L.usp_attn_fwd(qd, kd, vd, s_valid=s_valid, cu_seqlens=cu, causal=causal,
                                workspace=ws1)
    torch.cuda.synchronize()
    q64, k64, v64 = (f64(t) for t in (q, k, v))
    o, lse = oracle.attn_fwd(q64, k64, v64, d ** -0.5, s_valid, cu, causal)
    check_close("O (split)", f64(o_s), o, "bf16")
    check_close("LSE (split)", f64(lse_s), lse, "bf16")
    check_close("O (one pass)", f64(o_1), o, "bf16")
    check_close("LSE (one pass)", f64(lse_1), lse, "bf16")
    # backward from the split forward's O and LSE, dQ split and in one pass
    wsb, wsb1 = bwd_workspaces(L, s, s, hq, hkv, d, dev)
    assert L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, causal=causal,
                                     s_k_valid=s_valid, workspace_bytes=wsb1.numel()) == 1
    grads = {}
    for tag, ws in (("split", wsb), ("one pass", wsb1)):
        grads[tag] = L.usp_attn_bwd(qd, kd, vd, o_s, lse_s, dod, s_valid=s_valid, cu_seqlens=cu,
                                    causal=causal, workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = oracle.attn_bwd(q64, k64, v64, o, lse, f64(do), d ** -0.5, s_valid, cu, causal)
    for tag, (gq, gk, gv) in grads.items():
        check_close(f"dQ ({tag})", f64(gq), dq, "bf16")
        check_close(f"dK ({tag})", f64(gk), dk, "bf16")
        check_close(f"dV ({tag})", f64(gv), dv, "bf16")
    # dK and dV do not depend on the dQ plan
    assert torch.equal(grads["split"][1], grads["one pass"][1])
    assert torch.equal(grads["split"][2], grads["one pass"][2])


def test_split_forward_8k_sampled_rows():
    """The 8K share of a 4 Q / 1 KV head, d = 128 model: sampled rows, the first
    and last rows and the rows around each 64-row query block edge near the
    split boundaries."""
    L = usp()
    dev = gpu()
    s, hq, hkv, d = 8192, 4, 1, 128
    n = L.usp_attn_fwd_num_splits(s, s, hq, hkv, d, L.USP_BF16)
    nb = L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16)
    say(f"splits 8k: fwd splits={n} dq splits={nb}")
    assert n > 1 and nb > 1
    q, k, v, do = (seeded((s, h, d), 3000 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o_s, lse_s = L.usp_attn_fwd(qd, kd, vd)
    ws1 = torch.empty(vcopy_bytes(s, hkv, d), dtype=torch.uint8, device=dev)
    o_1, lse_1 = L.usp_attn_fwd(qd, kd, vd, workspace=ws1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = set(rng.choice(s, 160, replace=False).tolist())
    rows.update(range(0, 8))
    rows.update(range(s - 8, s))
    for b in range(1, 8):  # rows around key positions b * s / 8
        rows.update(range(b * s // 8 - 3, b * s // 8 + 3))
    rows = np.array(sorted(rows), dtype=np.int64)
    o_ref, lse_ref = oracle.attn_fwd_rows(f64(q), f64(k), f64(v), rows, d ** -0.5)
    check_close("O[rows] (split)", f64(o_s)[rows], o_ref, "bf16")
    check_close("LSE[rows] (split)", f64(lse_s)[:, rows], lse_ref, "bf16")
    check_close("O[rows] (one pass)", f64(o_1)[rows], o_ref, "bf16")
    check_close("LSE[rows] (one pass)", f64(lse_1)[:, rows], lse_ref, "bf16")
    # the two paths agree over every row, not only the sampled ones
    check_close("O split vs one pass", f64(o_s), f64(o_1), "bf16")
    assert np.isfinite(f64(lse_s)).all()
    wsb, wsb1 = bwd_workspaces(L, s, s, hq, hkv, d, dev)
    dq_s = L.usp_attn_bwd(qd, kd, vd, o_s, lse_s, dod, workspace=wsb)[0]
    dq_1 = L.usp_attn_bwd(qd, kd, vd, o_s, lse_s, dod, workspace=wsb1)[0]
    torch.cuda.synchronize()
    dq_ref = oracle.attn_bwd_rows(f64(q), f64(k), f64(v), f64(do), rows, d ** -0.5)
    check_close("dQ[rows] (split)", f64(dq_s)[rows], dq_ref, "bf16")
    check_close("dQ[rows] (one pass)", f64(dq_1)[rows], dq_ref, "bf16")
    check_close("dQ split vs one pass", f64(dq_s), f64(dq_1), "bf16")


INTERVAL = [
    # name, s_q, q_off, s_k, k_off, s_k_valid, hq, hkv, d, causal, cu (global), out dtype
    ("rows_after_keys", 1500, 2000, 3500, 0, 3500, 4, 1, 128, True, None, torch.float32),
    ("more_rows_than_keys_bidir", 3000, 0, 1000, 500, 990, 4, 1, 128, False, None, torch.bfloat16),
    ("second_half_gqa4_d64", 2500, 2500, 2500, 0, 2500, 8, 2, 64, True, None, torch.float32),
    ("docs_global", 2000, 2500, 5000, 0, 5000, 4, 1, 128, True, [0, 1200, 2600, 5000],
     torch.float32),
    # the first 1000 rows precede every key: O = 0, LSE = -inf
    ("rows_before_keys", 3000, 0, 3000, 1000, 3000, 4, 1, 128, True, None, torch.float32),
]


@pytest.mark.parametrize("case", INTERVAL, ids=[c[0] for c in INTERVAL])
def test_split_interval_forward(case):
    name, s_q, q_off, s_k, k_off, s_kv, hq, hkv, d, causal, cu, odt = case
    L = usp()
    dev = gpu()
    n = L.usp_attn_fwd_num_splits(s_q, s_k, hq, hkv, d, L.USP_BF16, causal=causal, q_off=q_off,
                                  k_off=k_off, s_k_valid=s_kv)
    nb = L.usp_attn_bwd_num_splits(s_q, s_k, hq, hkv, d, L.USP_BF16, causal=causal, q_off=q_off,
                                   k_off=k_off, s_k_valid=s_kv)
    say(f"split interval {name}: s_q={s_q}@{q_off} s_k={s_k}@{k_off} valid={s_kv} hq={hq} "
        f"hkv={hkv} d={d} causal={causal} fwd splits={n} dq splits={nb}")
    assert n > 1 and nb > 1
    q, do = (seeded((s_q, hq, d), 4000 + 3 * i) for i in range(2))
    k, v = (seeded((s_k, hkv, d), 4001 + i) for i in range(2))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    kw = dict(q_off=q_off, k_off=k_off, s_k_valid=s_kv, cu_seqlens=cu, causal=causal,
              out_dtype=odt)
    o_s, lse_s = L.usp_attn_fwd_interval(qd, kd, vd, **kw)
    ws1 = torch.empty(vcopy_bytes(s_k, hkv, d), dtype=torch.uint8, device=dev)
    o_1, lse_1 = L.usp_attn_fwd_interval(qd, kd, vd, workspace=ws1, **kw)
    torch.cuda.synchronize()
    o, lse = oracle.attn_fwd_partial(f64(q), f64(k), f64(v), d ** -0.5, q_off, k_off, s_kv, cu,
                                     causal)
    empty = np.isneginf(lse)
    for tag, og, lg in (("split", o_s, lse_s), ("one pass", o_1, lse_1)):
        lg64 = f64(lg)
        # rows with no allowed key: exactly O = 0, LSE = -inf
        assert (np.isneginf(lg64) == empty).all(), tag
        assert (f64(og).transpose(1, 0, 2)[empty] == 0).all(), tag
        check_close(f"O ({tag})", f64(og), o, "bf16", bf16_out=odt == torch.bfloat16)
        check_close(f"LSE ({tag}, rows with keys)", lg64[~empty], lse[~empty], "bf16")
    # backward of this key interval from the oracle's O and LSE (as after a
    # ring's merge), fp32 gradients added to existing contents; a row without
    # keys here takes LSE 0, as if its keys lay in other intervals
    o_in = torch.from_numpy(o).to(torch.bfloat16).to(dev)
    lse_b = np.where(empty, 0.0, lse)
    lse_in = torch.from_numpy(lse_b).to(torch.float32).to(dev)
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd_partial(
        f64(q), f64(k), f64(v), f64(o_in), f64(lse_in), f64(do), d ** -0.5, q_off, k_off, s_kv, cu,
        causal)
    wsb, wsb1 = bwd_workspaces(L, s_q, s_k, hq, hkv, d, dev)
    base_q = seeded((s_q, hq, d), 4100, torch.float32)
    base_k = seeded((s_k, hkv, d), 4101, torch.float32)
    for tag, ws in (("split", wsb), ("one pass", wsb1)):
        dq, dk, dv = base_q.to(dev), base_k.to(dev), base_k.to(dev)
        L.usp_attn_bwd_interval(qd, kd, vd, o_in, lse_in, dod, q_off=q_off, k_off=k_off,
                                s_k_valid=s_kv, cu_seqlens=cu, causal=causal, accumulate=True,
                                dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        check_close(f"dQ accumulated ({tag})", f64(dq) - f64(base_q), dq_ref, "bf16", bf16_out=False)
        check_close(f"dK accumulated ({tag})", f64(dk) - f64(base_k), dk_ref, "bf16", bf16_out=False)
        check_close(f"dV accumulated ({tag})", f64(dv) - f64(base_k), dv_ref, "bf16", bf16_out=False)
