"""Pins for the fp64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: a hand-derived
worked example, torch's float64 scaled_dot_product_attention with autograd,
scipy's logsumexp, central finite differences, closed forms and exact
identities of the softmax.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

RTOL_LIB = 1e-10


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def mask_matrix(s, s_valid, cu, causal):
    """Boolean [S, S] allowed-key matrix, written out element by element."""
    doc = np.zeros(s, dtype=np.int64)
    if cu is not None:
        for k in range(len(cu) - 1):
            for j in range(cu[k], cu[k + 1]):
                doc[j] = k
    m = np.zeros((s, s), dtype=bool)
    for i in range(s):
        for j in range(s):
            ok = j < s_valid and doc[i] == doc[j]
            if causal:
                ok = ok and j <= i
            m[i, j] = ok
    return m


def torch_reference(q, k, v, do, scale, s_valid, cu, causal):
    """torch float64 SDPA on the CPU with an explicit boolean mask; KV heads
    repeated per group; gradients by autograd of L = sum(O * dO)."""
    s, hq, d = q.shape
    g = hq // k.shape[1]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(g, dim=1)
    vv = tv.repeat_interleave(g, dim=1)
    mask = torch.tensor(mask_matrix(s, s_valid, cu, causal))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), kk.transpose(0, 1), vv.transpose(0, 1),
        attn_mask=mask, scale=scale).transpose(0, 1)
    (o * torch.tensor(do)).sum().backward()
    # LSE from scipy on the masked score matrix built with torch's matmul
    z = (torch.einsum("ihd,jhd->hij", tq.detach(), kk.detach()) * scale).numpy()
    z = np.where(mask.numpy()[None], z, -np.inf)
    lse = scipy.special.logsumexp(z, axis=2)
    return (o.detach().numpy(), lse, tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


CASES = [
    # name, S, s_valid, hq, hkv, d, cu_seqlens, causal
    ("causal_mha", 70, 70, 2, 2, 16, None, True),
    ("causal_gqa2", 97, 97, 4, 2, 16, None, True),
    ("causal_gqa4_pad", 96, 93, 4, 1, 8, None, True),
    ("thd_gqa2", 120, 120, 4, 2, 16, [0, 17, 18, 60, 120], True),
    ("noncausal_pad", 64, 61, 4, 2, 16, None, False),
    ("noncausal_thd", 50, 50, 2, 1, 8, [0, 20, 50], False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_oracle_matches_torch_sdpa(case):
    name, s, s_valid, hq, hkv, d, cu, causal = case
    q, k, v, do = (rand((s, h, d), seed) for seed, h in
                   zip(range(4), (hq, hkv, hkv, hq)))
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle.attn_fwd(q, k, v, scale, s_valid, cu, causal)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, scale, s_valid, cu, causal)
    ro, rlse, rdq, rdk, rdv = torch_reference(q, k, v, do, scale, s_valid, cu, causal)
    np.testing.assert_allclose(o, ro, rtol=RTOL_LIB, atol=RTOL_LIB)
    np.testing.assert_allclose(lse, rlse, rtol=RTOL_LIB, atol=RTOL_LIB)
    np.testing.assert_allclose(dq, rdq, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dk, rdk, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dv, rdv, rtol=1e-9, atol=1e-10)


def test_oracle_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "attn_worked_example.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        col = lambda a: np.asarray(a, dtype=np.float64).reshape(-1, 1, 1)
        q, k, v, do = col(c["q"]), col(c["k"]), col(c["v"]), col(c["do"])
        o, lse = oracle.attn_fwd(q, k, v, 1.0, c["s_valid"], c["cu_seqlens"], c["causal"])
        dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, 1.0, c["s_valid"],
                                     c["cu_seqlens"], c["causal"])
        np.testing.assert_allclose(o.ravel(), c["o"], atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(lse.ravel(), c["lse"], atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(dq.ravel(), c["dq"], atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(dk.ravel(), c["dk"], atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(dv.ravel(), c["dv"], atol=1e-14, err_msg=c["name"])


@pytest.mark.parametrize("cu,s_valid", [(None, 48), (None, 45), ([0, 20, 21, 48], 48)])
def test_oracle_finite_differences(cu, s_valid):
    s, hq, hkv, d = 48, 4, 2, 16
    q, k, v, do = (rand((s, h, d), 10 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    scale = 1.0 / np.sqrt(d)

    def loss(q_, k_, v_):
        o_, _ = oracle.attn_fwd(q_, k_, v_, scale, s_valid, cu)
        return float((o_ * do).sum())

    o, lse = oracle.attn_fwd(q, k, v, scale, s_valid, cu)
    grads = oracle.attn_bwd(q, k, v, o, lse, do, scale, s_valid, cu)
    eps = 1e-5
    g = np.random.default_rng(99)
    for which, x in enumerate((q, k, v)):
        for _ in range(12):
            idx = tuple(int(g.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            an = grads[which][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, idx, fd, an)


def test_closed_form_first_rows_and_doc_starts():
    s, hq, hkv, d = 64, 4, 2, 16
    cu = [0, 10, 11, 40, 64]
    q, k, v = (rand((s, h, d), 20 + i) for i, h in enumerate((hq, hkv, hkv)))
    scale = 0.25
    o, lse = oracle.attn_fwd(q, k, v, scale, s, cu)
    for start in cu[:-1]:
        for h in range(hq):
            np.testing.assert_array_equal(o[start, h], v[start, h // 2])
            assert lse[h, start] == pytest.approx(scale * q[start, h] @ k[start, h // 2], abs=1e-13)


def test_closed_form_zero_keys_mean_of_values():
    s, hq, hkv, d, s_valid = 40, 2, 1, 8, 37
    q, v = rand((s, hq, d), 30), rand((s, hkv, d), 31)
    k = np.zeros((s, hkv, d))
    o, lse = oracle.attn_fwd(q, k, v, 1.0, s_valid)
    for i in range(s):
        n = min(i, s_valid - 1) + 1
        for h in range(hq):
            np.testing.assert_allclose(o[i, h], v[:n, 0].mean(axis=0), atol=1e-13)
            assert lse[h, i] == pytest.approx(np.log(n), abs=1e-13)
    # packed documents: the mean runs over the document prefix only
    cu = [0, 15, 40]
    o, lse = oracle.attn_fwd(q, k, v, 1.0, s, cu)
    for i in range(s):
        st = 0 if i < 15 else 15
        np.testing.assert_allclose(o[i, 0], v[st:i + 1, 0].mean(axis=0), atol=1e-13)
        assert lse[0, i] == pytest.approx(np.log(i + 1 - st), abs=1e-13)


def test_closed_form_constant_values():
    s, hq, hkv, d = 33, 4, 2, 8
    q, k = rand((s, hq, d), 40), rand((s, hkv, d), 41)
    v = np.full((s, hkv, d), 0.375)
    o, _ = oracle.attn_fwd(q, k, v, 0.3, 30, [0, 5, 33])
    np.testing.assert_allclose(o, 0.375, atol=1e-14)


def test_padded_query_row_is_mean_of_valid_values():
    s, s_valid, d = 24, 21, 8
    q = rand((s, 2, d), 50)
    q[s_valid:] = 0.0  # pack zero-fills padded rows
    k, v = rand((s, 1, d), 51), rand((s, 1, d), 52)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, s_valid)
    for i in range(s_valid, s):
        np.testing.assert_allclose(o[i, :], np.broadcast_to(v[:s_valid, 0].mean(0), (2, d)), atol=1e-13)
        np.testing.assert_allclose(lse[:, i], np.log(s_valid), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_and_group_sums():
    s, hq, hkv, d, g = 50, 6, 2, 8, 3
    q, k, v, do = (rand((s, h, d), 60 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    o, lse = oracle.attn_fwd(q, k, v, 0.4)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, 0.4)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o2, lse2 = oracle.attn_fwd(q, kr, vr, 0.4)
    dq2, dk2, dv2 = oracle.attn_bwd(q, kr, vr, o2, lse2, do, 0.4)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(s, hkv, g, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(s, hkv, g, d).sum(2), atol=1e-13)


@pytest.mark.parametrize("cu,s_valid", [(None, 80), (None, 77), ([0, 30, 31, 80], 80)])
def test_gradient_identities(cu, s_valid):
    s, hq, hkv, d = 80, 4, 2, 16
    q, k, v, do = (rand((s, h, d), 70 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    o, lse = oracle.attn_fwd(q, k, v, 0.25, s_valid, cu)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, 0.25, s_valid, cu)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.reshape(s, hkv, 2, d).sum(axis=(0, 2)), atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals dO_i . O_i
    assert np.isfinite(dq).all()


def test_sampled_rows_and_keys_match_full():
    s, hq, hkv, d = 300, 4, 1, 16
    cu = [0, 100, 101, 260, 300]
    q, k, v, do = (rand((s, h, d), 80 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    for cu_, sv in ((None, 297), (cu, 300)):
        o, lse = oracle.attn_fwd(q, k, v, 0.25, sv, cu_)
        dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, 0.25, sv, cu_)
        rows = np.array([0, 1, 99, 100, 101, 150, 259, 260, 296, 297, 299])
        o_r, lse_r = oracle.attn_fwd_rows(q, k, v, rows, 0.25, sv, cu_)
        np.testing.assert_allclose(o_r, o[rows], atol=1e-13)
        np.testing.assert_allclose(lse_r, lse[:, rows], atol=1e-13)
        dq_r = oracle.attn_bwd_rows(q, k, v, do, rows, 0.25, sv, cu_)
        np.testing.assert_allclose(dq_r, dq[rows], atol=1e-12)
        dq_r = oracle.attn_bwd_rows(q, k, v, do, rows, 0.25, sv, cu_, lse=lse[:, rows])
        np.testing.assert_allclose(dq_r, dq[rows], atol=1e-12)
        keys = np.array([5, 99, 100, 200, 259, 280, 296, 297, 299])
        dk_r, dv_r = oracle.attn_bwd_keys(q, k, v, do, keys, 0.25, sv, cu_)
        np.testing.assert_allclose(dk_r, dk[keys], atol=1e-12)
        np.testing.assert_allclose(dv_r, dv[keys], atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    """A dropped D term or a transposed head mapping in the oracle must fail
    the library comparison (the mistake is planted in the oracle, on the CPU)."""
    case = CASES[1]
    _, s, s_valid, hq, hkv, d, cu, causal = case
    q, k, v, do = (rand((s, h, d), seed) for seed, h in zip(range(4), (hq, hkv, hkv, hq)))
    scale = 1.0 / np.sqrt(d)
    ref = torch_reference(q, k, v, do, scale, s_valid, cu, causal)
    import oracle.attention as A

    orig = A._bwd_block

    def no_d(*args):
        c0, nc, p, ds = orig(*args)
        q_, k_, v_, do_, h, kvh, rb = args[:7]
        dp = do_[rb, h, :] @ v_[c0:nc, kvh, :].T
        return c0, nc, p, p * dp  # D dropped

    monkeypatch.setattr(A, "_bwd_block", no_d)
    o, lse = oracle.attn_fwd(q, k, v, scale, s_valid, cu, causal)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, scale, s_valid, cu, causal)
    assert not np.allclose(dq, ref[2], atol=1e-6)
    monkeypatch.setattr(A, "_bwd_block", orig)

    orig_scores = A._scores

    def wrong_group(q_, k_, h, kvh, *rest):
        return orig_scores(q_, k_, h, h % k_.shape[1], *rest)  # h % hkv instead of h // g

    monkeypatch.setattr(A, "_scores", wrong_group)
    o, lse = oracle.attn_fwd(q, k, v, scale, s_valid, cu, causal)
    assert not np.allclose(o, ref[0], atol=1e-6)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sampled_keys_of_a_query_interval_match_torch(case):
    """attn_bwd_keys over a query interval [q_lo, q_hi) is that interval's
    contribution to dK / dV: the gradient of sum over the interval's rows of
    O * dO, i.e. torch autograd with dO set to zero outside the interval."""
    name, s, s_valid, hq, hkv, d, cu, causal = case
    q, k, v, do = (rand((s, h, d), 90 + seed) for seed, h in zip(range(4), (hq, hkv, hkv, hq)))
    scale = 1.0 / np.sqrt(d)
    keys = np.array(sorted({0, 1, 2, s // 3, s // 2, s - 5, s - 2, s - 1}))
    for q_lo, q_hi in ((0, s), (s // 4, s), (s // 3, 2 * s // 3), (s - 1, s)):
        do_i = np.zeros_like(do)
        do_i[q_lo:q_hi] = do[q_lo:q_hi]
        _, _, _, rdk, rdv = torch_reference(q, k, v, do_i, scale, s_valid, cu, causal)
        dk, dv = oracle.attn_bwd_keys(q, k, v, do, keys, scale, s_valid, cu, causal,
                                      q_lo=q_lo, q_hi=q_hi)
        np.testing.assert_allclose(dk, rdk[keys], atol=RTOL_LIB)
        np.testing.assert_allclose(dv, rdv[keys], atol=RTOL_LIB)


def test_sampled_key_absolute_sums_by_brute_force():
    """attn_bwd_keys(with_abs=True): the absolute-term sums written out with
    explicit loops over rows, keys and heads from their definitions
    (P from the textbook softmax, dS = P (dP - D), D = dO . O)."""
    import math
    s, hq, hkv, d = 12, 4, 2, 3
    cu, s_valid, scale = [0, 5, 12], 11, 0.7
    q, k, v, do = (rand((s, h, d), 140 + i) for i, h in enumerate((hq, hkv, hkv, hq)))
    g = hq // hkv
    doc = [0] * 5 + [1] * 7

    def allowed(i, j):
        return j < s_valid and j <= i and doc[i] == doc[j]

    P = np.zeros((hq, s, s))
    for h in range(hq):
        for i in range(s):
            zs = {j: scale * sum(q[i, h, e] * k[j, h // g, e] for e in range(d))
                  for j in range(s) if allowed(i, j)}
            tot = sum(math.exp(z) for z in zs.values())
            for j, z in zs.items():
                P[h, i, j] = math.exp(z) / tot
    keys = np.array([0, 3, 5, 6, 10, 11])
    want_dk = np.zeros((len(keys), hkv, d))
    want_adk = np.zeros((len(keys), hkv, d))
    want_adv = np.zeros((len(keys), hkv, d))
    for h in range(hq):
        for i in range(s):
            o_i = [sum(P[h, i, l] * v[l, h // g, e] for l in range(s)) for e in range(d)]
            oabs_i = [sum(P[h, i, l] * abs(v[l, h // g, e]) for l in range(s)) for e in range(d)]
            D = sum(do[i, h, e] * o_i[e] for e in range(d))
            B = sum(abs(do[i, h, e]) * oabs_i[e] for e in range(d))
            for a, j in enumerate(keys):
                if not allowed(i, j):
                    continue
                dp = sum(do[i, h, e] * v[j, h // g, e] for e in range(d))
                ds = P[h, i, j] * (dp - D)
                for e in range(d):
                    want_dk[a, h // g, e] += scale * ds * q[i, h, e]
                    want_adk[a, h // g, e] += scale * abs(q[i, h, e]) * (abs(ds) + P[h, i, j] * B)
                    want_adv[a, h // g, e] += P[h, i, j] * abs(do[i, h, e])
    dk, dv, adk, adv = oracle.attn_bwd_keys(q, k, v, do, keys, scale, s_valid, cu, True,
                                            with_abs=True)
    np.testing.assert_allclose(dk, want_dk, atol=1e-12)
    np.testing.assert_allclose(adk, want_adk, atol=1e-12)
    np.testing.assert_allclose(adv, want_adv, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sampled_key_absolute_sums_bound_the_values(case):
    """Triangle inequality: |dK| <= AdK and |dV| <= AdV element-wise; a key
    seen by one row of one head (the last key of a causal MHA sequence) has
    AdV = |dV| exactly."""
    name, s, s_valid, hq, hkv, d, cu, causal = case
    q, k, v, do = (rand((s, h, d), 150 + seed) for seed, h in zip(range(4), (hq, hkv, hkv, hq)))
    keys = np.arange(s)
    dk, dv, adk, adv = oracle.attn_bwd_keys(q, k, v, do, keys, 1.0 / np.sqrt(d), s_valid, cu,
                                            causal, with_abs=True)
    assert (np.abs(dk) <= adk + 1e-12).all() and (np.abs(dv) <= adv + 1e-12).all()
    if name == "causal_mha":
        np.testing.assert_allclose(adv[-1], np.abs(dv[-1]), rtol=1e-12)
