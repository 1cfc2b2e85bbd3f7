"""Pins for the oracle's pad + pack / unpack and the sequence-parallel
invariant (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_pack_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "pack_worked_example.json")) as f:
        fx = json.load(f)
    x = np.asarray(fx["x"], dtype=np.int64)
    y = oracle.pad_pack_seq2head(x, fx["p"])
    assert y.shape[1] == fx["s_pad"] == oracle.padded_len(x.shape[0], fx["p"])
    np.testing.assert_array_equal(y, np.asarray(fx["y"]))
    np.testing.assert_array_equal(oracle.unpack_head2seq(y, x.shape[0]), x)


def test_padded_len_values():
    # 119,999 tokens over 8 ranks pad to 120,000 (15,000 per slice)
    assert oracle.padded_len(119999, 8) == 120000
    assert oracle.padded_len(120000, 8) == 120000
    assert oracle.padded_len(131072, 2) == 131072
    assert oracle.padded_len(1, 8) == 8
    assert oracle.padded_len(0, 4) == 0
    with pytest.raises(ValueError):
        oracle.padded_len(5, 0)


def simulated_all_to_all(x, p):
    """Every rank packs its own slice into a send buffer; the all-to-all
    hands chunk dst of every source to rank dst. Explicit loops over ranks
    and rows, independent of the oracle's vectorised form."""
    s_real, h, d = x.shape
    s_pad = -(-s_real // p) * p
    s_loc, hp = s_pad // p, h // p
    xp = np.zeros((s_pad, h, d), dtype=x.dtype)
    for s in range(s_real):
        xp[s] = x[s]
    send = [[None] * p for _ in range(p)]
    for src in range(p):
        local = xp[src * s_loc:(src + 1) * s_loc]
        for dst in range(p):
            send[src][dst] = local[:, dst * hp:(dst + 1) * hp, :]
    recv = np.zeros((p, s_pad, hp, d), dtype=x.dtype)
    for dst in range(p):
        for src in range(p):
            recv[dst, src * s_loc:(src + 1) * s_loc] = send[src][dst]
    return recv


@pytest.mark.parametrize("s,h,p", [(16, 8, 2), (13, 8, 4), (7, 6, 3), (9, 4, 1), (1, 8, 8)])
def test_pack_equals_simulated_all_to_all(s, h, p):
    x = np.random.default_rng(s * 100 + h).integers(0, 1 << 16, (s, h, 5)).astype(np.uint16)
    y = oracle.pad_pack_seq2head(x, p)
    np.testing.assert_array_equal(y, simulated_all_to_all(x, p))
    s_pad = oracle.padded_len(s, p)
    assert (y[:, s:s_pad] == 0).all()
    back = oracle.unpack_head2seq(y, s)
    assert back.dtype == x.dtype
    np.testing.assert_array_equal(back, x)
    if p == 1:
        np.testing.assert_array_equal(y[0], x)


def test_pack_rejects_indivisible_heads():
    with pytest.raises(ValueError):
        oracle.pad_pack_seq2head(np.zeros((4, 6, 2)), 4)


def test_sequence_parallel_invariant_tiny():
    """The pages' parity test: Ulysses-sharded attention (pack, local
    attention on each rank's heads over the full sequence, unpack) equals
    full-sequence attention, for the output and every gradient. The
    full-sequence side is torch's float64 SDPA with autograd."""
    w = workloads.WORKLOADS["tiny"]
    s = 160  # shortened from 512 to keep the CPU suite fast; same shape otherwise
    q, k, v, do = (workloads.tensor(w, t, s=s).double().numpy()
                   for t in (workloads.Q, workloads.K, workloads.V, workloads.DO))
    p, scale = w.p, w.scale
    yq, yk, yv, ydo = (oracle.pad_pack_seq2head(a, p) for a in (q, k, v, do))
    outs = {n: [] for n in ("o", "dq", "dk", "dv")}
    for r in range(p):
        o_r, lse_r = oracle.attn_fwd(yq[r], yk[r], yv[r], scale)
        dq_r, dk_r, dv_r = oracle.attn_bwd(yq[r], yk[r], yv[r], o_r, lse_r, ydo[r], scale)
        for n, a in zip(("o", "dq", "dk", "dv"), (o_r, dq_r, dk_r, dv_r)):
            outs[n].append(a)
    got = {n: oracle.unpack_head2seq(np.stack(a), s) for n, a in outs.items()}

    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    g = w.hq_full // w.hkv_full
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), tk.repeat_interleave(g, 1).transpose(0, 1),
        tv.repeat_interleave(g, 1).transpose(0, 1), is_causal=True, scale=scale).transpose(0, 1)
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(got["o"], o.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(got["dq"], tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dk"], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dv"], tv.grad.numpy(), atol=1e-11)
    loss_sp = float((got["o"] * do).sum())
    loss_full = float((o.detach().numpy() * do).sum())
    assert loss_sp == pytest.approx(loss_full, abs=1e-10)


def test_workload_document_lengths():
    # seeded packed-document lengths for the 131,072-token workload
    lens = workloads.doc_lengths(131072)
    assert lens == [22017, 30947, 29985, 25197, 17499, 5427]
    cu = workloads.cu_seqlens(lens)
    assert cu.tolist() == [0, 22017, 52964, 82949, 108146, 125645, 131072]
    assert sum(L * (L + 1) // 2 for L in lens) == 1656126267
