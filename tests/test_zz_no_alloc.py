"""GPU check of usp_attn_bwd_noalloc (the backward with the library's static
workspace, for callers that cannot allocate): through the C ABI, against
usp_attn_bwd given a caller workspace of the same size (the same plan, so
the same kernels and the same bits), and against the fp64 oracle on the
smaller calls. Several calls in a row on one GPU, each smaller than the one
before, so that every call finds the previous call's data in the array."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, f64, gpu, say

pytestmark = pytest.mark.gpu


def seeded(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


CALLS = [
    # S, s_valid, hq, hkv, cu_seqlens; in this order, each smaller than the last
    (16384, 16384, 32, 8, [0, 5000, 5001, 12000, 16384]),  # one row chunk, no dQ key
                                                 # splits, longest-first block order
    (16320, 16320, 32, 8, None),                 # one row chunk, no dQ key splits
    (1000, 997, 4, 1, None),                     # 16 row chunks, dQ key splits, padding
    (777, 777, 8, 2, [0, 300, 301, 777]),        # 2 row chunks, documents
]


def test_noalloc_backward_matches_usp_attn_bwd_on_successive_calls():
    import ulysses_sequence_parallelism_amd as L
    dev = gpu()
    d = 128
    for n, (s, s_valid, hq, hkv, cu) in enumerate(CALLS):
        say(f"call {n}: S={s} s_valid={s_valid} hq={hq} hkv={hkv} docs={cu}")
        need = L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16)
        q, k, v, do = (seeded((s, h, d), [17, n, i]) for i, h in enumerate((hq, hkv, hkv, hq)))
        if s_valid < s:
            for t in (q, k, v, do):
                t[s_valid:] = 0
        qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
        o, lse = L.usp_attn_fwd(qd, kd, vd, s_valid=s_valid, cu_seqlens=cu)
        # the caller-workspace call with exactly the static array's room: same plan
        ws = torch.empty(L.USP_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
        ref = L.usp_attn_bwd(qd, kd, vd, o, lse, dod, s_valid=s_valid, cu_seqlens=cu, workspace=ws)
        assert L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, s_k_valid=s_valid,
                                         workspace_bytes=ws.numel()) >= 1
        del ws
        torch.cuda.synchronize()
        # outputs preallocated and filled with garbage: the call must overwrite them
        got = tuple(torch.full_like(t, float("nan")) for t in ref)
        cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
        L.usp_trace_collect()
        L.usp_trace_enable(True)
        try:
            L.usp_attn_bwd_noalloc(qd, kd, vd, o, lse, dod, s_valid=s_valid, cu_seqlens=cu_dev,
                                   dq=got[0], dk=got[1], dv=got[2])
            torch.cuda.synchronize()
            ran = {e["name"]: e["launches"] for e in L.usp_trace_collect()}
        finally:
            L.usp_trace_enable(False)
        # the order tables of the dK/dV and dQ grids live in the static array too
        if n == 0:
            assert ran.get("attn_block_order") == 2, ran
        say(f"  required workspace {need} bytes")
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {n} {name} differs"
        if s <= 1000:
            q64, k64, v64, do64 = (f64(t) for t in (q, k, v, do))
            ro, rlse = oracle.attn_fwd(q64, k64, v64, d ** -0.5, s_valid, cu)
            rdq, rdk, rdv = oracle.attn_bwd(q64, k64, v64, ro, rlse, do64, d ** -0.5, s_valid, cu)
            check_close("dQ", f64(got[0]), rdq, "bf16")
            check_close("dK", f64(got[1]), rdk, "bf16")
            check_close("dV", f64(got[2]), rdv, "bf16")


def test_noalloc_backward_rejects_sizes_beyond_the_array():
    import ulysses_sequence_parallelism_amd as L
    dev = gpu()
    s, hq, hkv, d = 8192, 4, 1, 128   # 16 row chunks of partial dK / dV: 134 MB
    assert L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16) > L.USP_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((s, hq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((s, hkv, d), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((hq, s), dtype=torch.float32, device=dev)
    with pytest.raises(L.UspError) as e:
        L.usp_attn_bwd_noalloc(q, k, k.clone(), q.clone(), lse, q.clone())
    assert e.value.status == -5
