"""Oracle: exact grouped-query attention, forward and backward, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed. After the Ulysses all-to-all each rank runs ordinary local
attention over the FULL sequence for its share of heads, with separate query
and key/value head counts ("feat(dspark): add Ulysses sequence parallel
training", Modifications); gradients flow through that path and are checked
against a full-sequence reference (same page, Accuracy Test). For query head h
the key/value head is h // g with g = Hq / Hkv. For query row i the allowed
key set is

    M(i) = { j : j < S_valid,  j <= i (causal),  doc(j) == doc(i) }

where doc() comes from packed-sequence offsets cu_seqlens ("GLM-5.2 131k
context parallelism", Purpose: THD packed sequences with cu_seqlens) and
S_valid masks the alignment padding (readings: causal with the diagonal
included; padded keys masked; padded queries computed like any other row).
With z_ij = scale * q_i . k_j:

    LSE_i = log sum_{j in M(i)} exp(z_ij)
    O_i   = sum_{j in M(i)} exp(z_ij - LSE_i) v_j

Backward, for the loss L with dL/dO = dO (chain rule through the softmax):

    P_ij  = exp(z_ij - LSE_i)   (0 off M(i))
    dP_ij = dO_i . v_j
    D_i   = sum_j P_ij dP_ij
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_{h in group} sum_i dS_ij q_i
    dV_j  = sum_{h in group} sum_i P_ij dO_i

Method: the textbook softmax over explicitly materialised score rows (one
block of query rows at a time, every allowed key at once): no online
rescaling, no tiling of the key axis. Matrix products are numpy's (a library
primitive); nothing else is fused or reordered.

Array layout: q, dO, O are [S_pad, Hq, d]; k, v are [S_pad, Hkv, d]; LSE is
[Hq, S_pad]. All float64 (bf16 inputs are up-cast exactly by the caller).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


def doc_of(n: int, cu_seqlens) -> np.ndarray | None:
    """doc(j) for j < n from offsets cu = [0, L0, L0+L1, ..., n]; None if no
    packing."""
    if cu_seqlens is None:
        return None
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != n or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at S")
    doc = np.empty(n, dtype=np.int64)
    for k in range(len(cu) - 1):
        doc[cu[k]:cu[k + 1]] = k
    return doc


def allowed_keys(rows: np.ndarray, ncols: int, s_valid: int, doc, causal: bool) -> np.ndarray:
    """Boolean [len(rows), ncols]: entry (a, j) is True iff key j is in M(rows[a])."""
    cols = np.arange(ncols)
    m = np.broadcast_to(cols[None, :] < s_valid, (len(rows), ncols)).copy()
    if causal:
        m &= cols[None, :] <= rows[:, None]
    if doc is not None:
        m &= doc[cols][None, :] == doc[rows][:, None]
    return m


def _check(q, k, v):
    s, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != s or k.shape[2] != d:
        raise ValueError("q, k, v shapes disagree")
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return s, hq, hkv, d, hq // hkv


def _scores(q, k, h, kvh, rows, ncols, scale, s_valid, doc, causal):
    """z for the given rows of head h against keys [0, ncols), with -inf off
    M(i)."""
    z = scale * (q[rows, h, :] @ k[:ncols, kvh, :].T)
    z[~allowed_keys(rows, ncols, s_valid, doc, causal)] = -np.inf
    return z


def _ncols(rows, s, causal):
    return int(rows.max()) + 1 if causal else s


def attn_fwd_rows(q, k, v, rows, scale, s_valid=None, cu_seqlens=None, causal=True):
    """O and LSE for the selected query rows only: ([len(rows), Hq, d],
    [Hq, len(rows)]). Each row costs O(S d)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), hq, d))
    lse = np.zeros((hq, len(rows)))
    for b0 in range(0, len(rows), ROW_BLOCK):
        rb = rows[b0:b0 + ROW_BLOCK]
        nc = _ncols(rb, s, causal)
        for h in range(hq):
            z = _scores(q, k, h, h // g, rb, nc, scale, s_valid, doc, causal)
            m = z.max(axis=1)
            l = np.exp(z - m[:, None]).sum(axis=1)
            lse_b = m + np.log(l)
            p = np.exp(z - lse_b[:, None])
            o[b0:b0 + len(rb), h, :] = p @ v[:nc, h // g, :]
            lse[h, b0:b0 + len(rb)] = lse_b
    return o, lse


def attn_fwd(q, k, v, scale, s_valid=None, cu_seqlens=None, causal=True):
    """Full forward: O [S, Hq, d] and LSE [Hq, S]."""
    s = np.asarray(q).shape[0]
    return attn_fwd_rows(q, k, v, np.arange(s), scale, s_valid, cu_seqlens, causal)


def _bwd_block(q, k, v, do, h, kvh, rb, lse_b, scale, s_valid, doc, causal, s):
    nc = _ncols(rb, s, causal)
    z = _scores(q, k, h, kvh, rb, nc, scale, s_valid, doc, causal)
    p = np.exp(z - lse_b[:, None])
    dp = do[rb, h, :] @ v[:nc, kvh, :].T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    return nc, p, ds


def attn_bwd(q, k, v, o, lse, do, scale, s_valid=None, cu_seqlens=None, causal=True):
    """Full backward: (dQ [S, Hq, d], dK [S, Hkv, d], dV [S, Hkv, d]).

    ``o`` is accepted for interface symmetry; D is the textbook row sum
    sum_j P_ij dP_ij, which equals dO_i . O_i."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    lse = np.asarray(lse, dtype=np.float64)
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b0 in range(0, s, ROW_BLOCK):
        rb = np.arange(b0, min(s, b0 + ROW_BLOCK))
        for h in range(hq):
            kvh = h // g
            nc, p, ds = _bwd_block(q, k, v, do, h, kvh, rb, lse[h, rb], scale,
                                   s_valid, doc, causal, s)
            dq[rb, h, :] = scale * (ds @ k[:nc, kvh, :])
            dk[:nc, kvh, :] += scale * (ds.T @ q[rb, h, :])
            dv[:nc, kvh, :] += p.T @ do[rb, h, :]
    return dq, dk, dv


def attn_bwd_rows(q, k, v, do, rows, scale, s_valid=None, cu_seqlens=None, causal=True):
    """dQ for the selected query rows only: [len(rows), Hq, d]. LSE of those
    rows is recomputed here, so no full forward is needed."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    rows = np.asarray(rows, dtype=np.int64)
    _, lse = attn_fwd_rows(q, k, v, rows, scale, s_valid, cu_seqlens, causal)
    dq = np.zeros((len(rows), hq, d))
    for b0 in range(0, len(rows), ROW_BLOCK):
        rb = rows[b0:b0 + ROW_BLOCK]
        for h in range(hq):
            nc, _, ds = _bwd_block(q, k, v, do, h, h // g, rb, lse[h, b0:b0 + len(rb)],
                                   scale, s_valid, doc, causal, s)
            dq[b0:b0 + len(rb), h, :] = scale * (ds @ k[:nc, h // g, :])
    return dq


def attn_bwd_keys(q, k, v, do, keys, scale, s_valid=None, cu_seqlens=None, causal=True):
    """dK and dV for the selected key rows only: ([len(keys), Hkv, d] x 2).

    Every query row i whose allowed set M(i) contains one of the keys is
    recomputed in full (LSE and D need the whole row), so this is cheap only
    when few rows see those keys, e.g. keys near the end of a causal
    sequence or of a document."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    keys = np.asarray(keys, dtype=np.int64)
    # rows that see at least one selected key
    cand = np.arange(int(keys.min()) if causal else 0, s)
    seen = np.zeros(len(cand), dtype=bool)
    for j0 in range(0, len(keys), 64):
        kj = keys[j0:j0 + 64]
        m = np.ones((len(cand), len(kj)), dtype=bool)
        m &= (kj < s_valid)[None, :]
        if causal:
            m &= kj[None, :] <= cand[:, None]
        if doc is not None:
            m &= doc[kj][None, :] == doc[cand][:, None]
        seen |= m.any(axis=1)
    rows = cand[seen]
    dk = np.zeros((len(keys), hkv, d))
    dv = np.zeros((len(keys), hkv, d))
    if len(rows) == 0:
        return dk, dv
    _, lse = attn_fwd_rows(q, k, v, rows, scale, s_valid, cu_seqlens, causal)
    for b0 in range(0, len(rows), ROW_BLOCK):
        rb = rows[b0:b0 + ROW_BLOCK]
        for h in range(hq):
            kvh = h // g
            nc, p, ds = _bwd_block(q, k, v, do, h, kvh, rb, lse[h, b0:b0 + len(rb)],
                                   scale, s_valid, doc, causal, s)
            sel = keys < nc
            ks = keys[sel]
            dk[sel, kvh, :] += scale * (ds[:, ks].T @ q[rb, h, :])
            dv[sel, kvh, :] += p[:, ks].T @ do[rb, h, :]
    return dk, dv
