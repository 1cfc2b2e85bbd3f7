"""GPU check that the library's calls can be captured in a HIP graph
(torch.cuda.CUDAGraph): a forward + backward is captured once and replayed
several times, each replay on new inputs written eagerly into the captured
buffers between replays, and each compared bit for bit with eager calls on the
same inputs. The calls enqueue kernels only (no memset or copy nodes), and
packed-document offsets go in as a device tensor, which the binding passes as
is."""
import pytest
import torch

from tests.gpu_helpers import gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, S, hq, hkv, cu_seqlens
    # forward key splits + merge, dK/dV row chunks + reduction, dQ key splits + reduction
    ("8k_splits_and_chunks", 8192, 4, 1, None),
    # the forward's longest-first block order (cost, rank with atomics, scatter)
    ("16k_docs_16q4kv", 16384, 16, 4, [0, 5000, 5001, 12000, 16384]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager_calls(case):
    import ulysses_sequence_parallelism_amd as L
    name, s, hq, hkv, cu = case
    dev = gpu()
    d = 128
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    q = torch.empty((s, hq, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((s, hkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    do = torch.empty_like(q)
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((hq, s), dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16),
                       dtype=torch.uint8, device=dev)

    def fill(seed):
        g = torch.Generator(device="cpu").manual_seed(seed)
        for t in (q, k, v, do):
            t.copy_(torch.randn(t.shape, generator=g).to(torch.bfloat16))

    def run():
        L.usp_attn_fwd(q, k, v, cu_seqlens=cu_dev, out=o, lse=lse, workspace=ws_f)
        L.usp_attn_bwd(q, k, v, o, lse, do, cu_seqlens=cu_dev, dq=dq, dk=dk, dv=dv,
                       workspace=ws_b)

    say(f"{name}: forward splits "
        f"{L.usp_attn_fwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, workspace_bytes=ws_f.numel())}, "
        f"dQ splits "
        f"{L.usp_attn_bwd_num_splits(s, s, hq, hkv, d, L.USP_BF16, workspace_bytes=ws_b.numel())}")
    # warm up on a side stream, then capture
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        fill(rep + 1)
        torch.cuda.synchronize()
        o_e, lse_e = L.usp_attn_fwd(q, k, v, cu_seqlens=cu_dev)
        dq_e, dk_e, dv_e = L.usp_attn_bwd(q, k, v, o_e, lse_e, do, cu_seqlens=cu_dev)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for tag, a, b in (("O", o, o_e), ("LSE", lse, lse_e), ("dQ", dq, dq_e), ("dK", dk, dk_e),
                          ("dV", dv, dv_e)):
            same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
            assert same, f"{name}: replay {rep} {tag} differs from the eager call"
        say(f"{name}: replay {rep} matches the eager calls bit for bit")
