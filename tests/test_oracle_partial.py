"""Pins for the oracle's interval attention, log-sum-exp merge and interval
backward (CPU only): splitting the key axis (ring / USP) or the query axis
(contiguous context parallelism) and recombining must reproduce full-sequence
attention, checked against torch's float64 SDPA with autograd."""
import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_full(q, k, v, do, scale, cu, causal, s_valid=None):
    s, hq, d = q.shape
    g = hq // k.shape[1]
    doc = np.zeros(s, dtype=np.int64)
    if cu is not None:
        for i in range(len(cu) - 1):
            doc[cu[i]:cu[i + 1]] = i
    idx = np.arange(s)
    mask = doc[:, None] == doc[None, :]
    if causal:
        mask &= idx[None, :] <= idx[:, None]
    if s_valid is not None:
        mask &= idx[None, :] < s_valid
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), tk.repeat_interleave(g, 1).transpose(0, 1),
        tv.repeat_interleave(g, 1).transpose(0, 1), attn_mask=torch.tensor(mask),
        scale=scale).transpose(0, 1)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


CASES = [
    # S, hq, hkv, key chunk edges, query chunk edges, cu_seqlens, causal
    (96, 4, 2, [0, 40, 41, 96], [0, 33, 96], None, True),
    (80, 4, 1, [0, 16, 32, 48, 64, 80], [0, 80], None, True),
    (90, 2, 2, [0, 45, 90], [0, 30, 60, 90], [0, 20, 57, 90], True),
    (64, 4, 2, [0, 20, 64], [0, 10, 64], None, False),
]


@pytest.mark.parametrize("case", CASES)
def test_interval_split_recombines_to_full_attention(case):
    s, hq, hkv, kedges, qedges, cu, causal = case
    d, scale = 16, 0.25
    q, k, v, do = (rand((s, h, d), 500 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    ro, rdq, rdk, rdv = torch_full(q, k, v, do, scale, cu, causal)
    o_full = np.zeros_like(q)
    lse_full = np.zeros((hq, s))
    for qa, qb in zip(qedges[:-1], qedges[1:]):
        parts = []
        for ka, kb in zip(kedges[:-1], kedges[1:]):
            parts.append(oracle.attn_fwd_partial(q[qa:qb], k[ka:kb], v[ka:kb], scale, q_off=qa,
                                                 k_off=ka, cu_seqlens=cu, causal=causal))
        o_m, lse_m = oracle.lse_merge(parts)
        o_full[qa:qb], lse_full[:, qa:qb] = o_m, lse_m
    np.testing.assert_allclose(o_full, ro, atol=1e-12)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, None, cu, causal)
    np.testing.assert_allclose(lse_full, lse_ref, atol=1e-12)
    # backward: dQ summed over key intervals, dK / dV over query intervals
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qa, qb in zip(qedges[:-1], qedges[1:]):
        for ka, kb in zip(kedges[:-1], kedges[1:]):
            a, b, c = oracle.attn_bwd_partial(q[qa:qb], k[ka:kb], v[ka:kb], o_full[qa:qb],
                                              lse_full[:, qa:qb], do[qa:qb], scale, q_off=qa,
                                              k_off=ka, cu_seqlens=cu, causal=causal)
            dq[qa:qb] += a
            dk[ka:kb] += b
            dv[ka:kb] += c
    np.testing.assert_allclose(dq, rdq, atol=1e-10)
    np.testing.assert_allclose(dk, rdk, atol=1e-10)
    np.testing.assert_allclose(dv, rdv, atol=1e-10)


def test_future_key_interval_gives_empty_rows():
    q, k, v = rand((8, 2, 4), 1), rand((6, 1, 4), 2), rand((6, 1, 4), 3)
    o, lse = oracle.attn_fwd_partial(q, k, v, 0.5, q_off=0, k_off=10)
    assert np.isneginf(lse).all() and (o == 0).all()
    # partly visible: rows 0..9 see nothing, later rows see a prefix
    o, lse = oracle.attn_fwd_partial(rand((14, 2, 4), 4), k, v, 0.5, q_off=0, k_off=10)
    assert np.isneginf(lse[:, :10]).all() and np.isfinite(lse[:, 10:]).all()
    # row 10 sees exactly key 0: O = v_0, LSE = scale q.k
    assert np.allclose(o[10, :, :], v[0, 0])


def test_lse_merge_identities():
    o, lse = rand((5, 2, 3), 7), rand((2, 5), 8)
    o2, lse2 = oracle.lse_merge([(o, lse)])
    np.testing.assert_allclose(o2, o)
    np.testing.assert_allclose(lse2, lse)
    empty = (np.zeros_like(o), np.full_like(lse, -np.inf))
    o3, lse3 = oracle.lse_merge([empty, (o, lse), empty])
    np.testing.assert_allclose(o3, o)
    np.testing.assert_allclose(lse3, lse)
    # two equal halves: LSE grows by log 2, O is unchanged
    o4, lse4 = oracle.lse_merge([(o, lse), (o, lse)])
    np.testing.assert_allclose(o4, o)
    np.testing.assert_allclose(lse4, lse + np.log(2.0))


def test_contiguous_query_interval_equals_rows_of_full_attention():
    """Contiguous context parallelism: a rank's query rows against the whole
    key sequence, with the causal offset, are the same rows of full attention."""
    s, hq, hkv, d = 120, 4, 2, 8
    q, k, v = (rand((s, h, d), 30 + i) for i, h in enumerate((hq, hkv, hkv)))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, 0.3)
    for qa, qb in ((0, 40), (40, 80), (80, 120), (57, 58)):
        o, lse = oracle.attn_fwd_partial(q[qa:qb], k, v, 0.3, q_off=qa, k_off=0)
        np.testing.assert_allclose(o, o_ref[qa:qb], atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref[:, qa:qb], atol=1e-13)


# Padded keys inside the intervals: with S_valid < S the last key block (or
# more) holds keys past the real sequence, which must be masked; the interval
# functions take that as sk_valid = the valid keys of the block. Padded query
# rows are computed like any other row.
PAD_CASES = [
    # S, S_valid, hq, hkv, key chunk edges, query chunk edges, causal
    (96, 90, 4, 2, [0, 40, 64, 96], [0, 33, 96], True),           # last block 26 of 32 valid
    (80, 70, 4, 1, [0, 16, 32, 48, 64, 80], [0, 40, 80], True),   # ring of 5, last block 6 of 16
    (50, 40, 2, 2, [0, 40, 50], [0, 25, 50], True),               # last block entirely padding
    (64, 60, 4, 2, [0, 20, 64], [0, 10, 64], False),
    (72, 65, 2, 1, [0, 64, 72], [0, 72], False),                  # last block with one valid key
]


@pytest.mark.parametrize("case", PAD_CASES)
def test_interval_split_with_padded_keys_recombines_to_full_attention(case):
    s, s_valid, hq, hkv, kedges, qedges, causal = case
    d, scale = 16, 0.3
    q, k, v, do = (rand((s, h, d), 600 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    ro, rdq, rdk, rdv = torch_full(q, k, v, do, scale, None, causal, s_valid=s_valid)
    o_full = np.zeros_like(q)
    lse_full = np.zeros((hq, s))
    for qa, qb in zip(qedges[:-1], qedges[1:]):
        parts = []
        for ka, kb in zip(kedges[:-1], kedges[1:]):
            skv = min(max(s_valid - ka, 0), kb - ka)
            o_p, lse_p = oracle.attn_fwd_partial(q[qa:qb], k[ka:kb], v[ka:kb], scale, q_off=qa,
                                                 k_off=ka, sk_valid=skv, causal=causal)
            if skv == 0:
                assert np.isneginf(lse_p).all() and (o_p == 0).all()
            parts.append((o_p, lse_p))
        o_full[qa:qb], lse_full[:, qa:qb] = oracle.lse_merge(parts)
    np.testing.assert_allclose(o_full, ro, atol=1e-12)
    _, lse_ref = oracle.attn_fwd(q, k, v, scale, s_valid, None, causal)
    np.testing.assert_allclose(lse_full, lse_ref, atol=1e-12)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qa, qb in zip(qedges[:-1], qedges[1:]):
        for ka, kb in zip(kedges[:-1], kedges[1:]):
            skv = min(max(s_valid - ka, 0), kb - ka)
            a, b, c = oracle.attn_bwd_partial(q[qa:qb], k[ka:kb], v[ka:kb], o_full[qa:qb],
                                              lse_full[:, qa:qb], do[qa:qb], scale, q_off=qa,
                                              k_off=ka, sk_valid=skv, causal=causal)
            dq[qa:qb] += a
            dk[ka:kb] += b
            dv[ka:kb] += c
    np.testing.assert_allclose(dq, rdq, atol=1e-10)
    np.testing.assert_allclose(dk, rdk, atol=1e-10)
    np.testing.assert_allclose(dv, rdv, atol=1e-10)
    # padded keys get no gradient at all
    assert (dk[s_valid:] == 0).all() and (dv[s_valid:] == 0).all()
