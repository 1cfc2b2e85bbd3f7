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


def _scores(q, k, h, kvh, rows, ncols, scale, s_valid, doc, causal, c0=0):
    """z for the given rows of head h against keys [c0, ncols), with -inf off
    M(i) (keys before c0 are outside every row's M(i))."""
    z = scale * (q[rows, h, :] @ k[c0:ncols, kvh, :].T)
    z[~allowed_keys(rows, ncols, s_valid, doc, causal)[:, c0:]] = -np.inf
    return z


def _ncols(rows, s, causal):
    return int(rows.max()) + 1 if causal else s


def _blocks(rows, doc):
    """Index ranges [a, b) of consecutive entries of `rows`, at most ROW_BLOCK
    long and, with documents, all in one document (so a block's keys start
    at that document's start)."""
    n = len(rows)
    if doc is None:
        return [(a, min(n, a + ROW_BLOCK)) for a in range(0, n, ROW_BLOCK)]
    d = doc[rows]
    cuts = [0] + [i for i in range(1, n) if d[i] != d[i - 1]] + [n]
    out = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        out += [(x, min(b, x + ROW_BLOCK)) for x in range(a, b, ROW_BLOCK)]
    return out


def _col0(rows, doc):
    """First key any of the rows may see: the start of the earliest row's
    document (0 without documents)."""
    if doc is None:
        return 0
    d0 = doc[int(rows.min())]
    return int(np.searchsorted(doc, d0))


def attn_fwd_rows(q, k, v, rows, scale, s_valid=None, cu_seqlens=None, causal=True,
                  with_abs=False):
    """O and LSE for the selected query rows only: ([len(rows), Hq, d],
    [Hq, len(rows)]). Each row costs O(S d).

    with_abs: also return sum_j P_ij |v_j| ([len(rows), Hq, d]), the sum of
    the absolute terms of O (its size when every term had the same sign)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), hq, d))
    lse = np.zeros((hq, len(rows)))
    oabs = np.zeros((len(rows), hq, d)) if with_abs else None
    for b0, b1 in _blocks(rows, doc):
        rb = rows[b0:b1]
        nc = _ncols(rb, s, causal)
        c0 = _col0(rb, doc)
        for h in range(hq):
            z = _scores(q, k, h, h // g, rb, nc, scale, s_valid, doc, causal, c0)
            m = z.max(axis=1)
            l = np.exp(z - m[:, None]).sum(axis=1)
            lse_b = m + np.log(l)
            p = np.exp(z - lse_b[:, None])
            o[b0:b0 + len(rb), h, :] = p @ v[c0:nc, h // g, :]
            lse[h, b0:b0 + len(rb)] = lse_b
            if with_abs:
                oabs[b0:b0 + len(rb), h, :] = p @ np.abs(v[c0:nc, h // g, :])
    return (o, lse, oabs) if with_abs else (o, lse)


def attn_fwd(q, k, v, scale, s_valid=None, cu_seqlens=None, causal=True):
    """Full forward: O [S, Hq, d] and LSE [Hq, S]."""
    s = np.asarray(q).shape[0]
    return attn_fwd_rows(q, k, v, np.arange(s), scale, s_valid, cu_seqlens, causal)


def _bwd_block(q, k, v, do, h, kvh, rb, lse_b, scale, s_valid, doc, causal, s):
    """P and dS of the rows rb of head h over keys [c0, nc)."""
    nc = _ncols(rb, s, causal)
    c0 = _col0(rb, doc)
    z = _scores(q, k, h, kvh, rb, nc, scale, s_valid, doc, causal, c0)
    p = np.exp(z - lse_b[:, None])
    dp = do[rb, h, :] @ v[c0:nc, kvh, :].T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    return c0, nc, p, ds


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
            c0, nc, p, ds = _bwd_block(q, k, v, do, h, kvh, rb, lse[h, rb], scale,
                                       s_valid, doc, causal, s)
            dq[rb, h, :] = scale * (ds @ k[c0:nc, kvh, :])
            dk[c0:nc, kvh, :] += scale * (ds.T @ q[rb, h, :])
            dv[c0:nc, kvh, :] += p.T @ do[rb, h, :]
    return dq, dk, dv


def attn_bwd_rows(q, k, v, do, rows, scale, s_valid=None, cu_seqlens=None, causal=True,
                  lse=None):
    """dQ for the selected query rows only: [len(rows), Hq, d]. The rows'
    LSE [Hq, len(rows)] is the oracle's own (attn_fwd_rows of the same rows,
    recomputed here when not given), so no full forward is needed."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    doc = doc_of(s, cu_seqlens)
    rows = np.asarray(rows, dtype=np.int64)
    if lse is None:
        _, lse = attn_fwd_rows(q, k, v, rows, scale, s_valid, cu_seqlens, causal)
    dq = np.zeros((len(rows), hq, d))
    for b0, b1 in _blocks(rows, doc):
        rb = rows[b0:b1]
        for h in range(hq):
            c0, nc, _, ds = _bwd_block(q, k, v, do, h, h // g, rb, lse[h, b0:b0 + len(rb)],
                                       scale, s_valid, doc, causal, s)
            dq[b0:b0 + len(rb), h, :] = scale * (ds @ k[c0:nc, h // g, :])
    return dq


def attn_bwd_keys(q, k, v, do, keys, scale, s_valid=None, cu_seqlens=None, causal=True,
                  q_lo=0, q_hi=None, with_abs=False):
    """dK and dV for the selected key rows only: ([len(keys), Hkv, d] x 2),
    from the query rows [q_lo, q_hi) (default: all rows; a smaller interval
    gives that interval's contribution, e.g. one ring or context-parallel
    rank's rows).

    Every query row of the interval whose allowed set M(i) contains one of
    the keys needs LSE_i and D_i = dO_i . O_i over its WHOLE row, so those
    rows are run through attn_fwd_rows first; the gradient terms are then
    formed for the selected key columns only:
        dK_j = scale sum_h sum_i P_ij (dP_ij - D_i) q_i,  dV_j = sum_h sum_i P_ij dO_i.

    with_abs: also return, per element, the sums of absolute values that
    bound how far rounding the factors of these terms can move them (the
    condition of each sum):
        AdK_j = scale sum_h sum_i |q_i| (|dS_ij| + P_ij B_i),
        AdV_j = sum_h sum_i P_ij |dO_i|,
    with B_i = sum_e |dO_ie| (sum_l P_il |v_le|), the bound of D_i's own
    sum. Returns (dK, dV, AdK, AdV)."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    s, hq, hkv, d, g = _check(q, k, v)
    s_valid = s if s_valid is None else s_valid
    q_hi = s if q_hi is None else q_hi
    doc = doc_of(s, cu_seqlens)
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((len(keys), hkv, d))
    dv = np.zeros((len(keys), hkv, d))
    adk = np.zeros((len(keys), hkv, d)) if with_abs else None
    adv = np.zeros((len(keys), hkv, d)) if with_abs else None
    out = (dk, dv, adk, adv) if with_abs else (dk, dv)
    # rows of the interval that see at least one selected key
    cand = np.arange(max(q_lo, int(keys.min()) if causal else q_lo), q_hi)
    if len(cand) == 0:
        return out
    seen = np.zeros(len(cand), dtype=bool)
    for r0 in range(0, len(cand), 4096):
        seen[r0:r0 + 4096] = _sees(cand[r0:r0 + 4096], keys, s_valid, doc, causal).any(axis=1)
    rows = cand[seen]
    if len(rows) == 0:
        return out
    fw = attn_fwd_rows(q, k, v, rows, scale, s_valid, cu_seqlens, causal, with_abs=with_abs)
    o, lse = fw[0], fw[1]
    dd = np.einsum("rhd,rhd->hr", do[rows], o)          # D_i = dO_i . O_i, [Hq, rows]
    if with_abs:
        bb = np.einsum("rhd,rhd->hr", np.abs(do[rows]), fw[2])   # B_i, [Hq, rows]
    for b0 in range(0, len(rows), ROW_BLOCK):
        rb = rows[b0:b0 + ROW_BLOCK]
        m = _sees(rb, keys, s_valid, doc, causal)          # [rows, keys]
        for h in range(hq):
            kvh = h // g
            z = scale * (q[rb, h, :] @ k[keys, kvh, :].T)
            p = np.where(m, np.exp(np.where(m, z, 0.0) - lse[h, b0:b0 + len(rb)][:, None]), 0.0)
            dp = do[rb, h, :] @ v[keys, kvh, :].T
            ds = p * (dp - dd[h, b0:b0 + len(rb)][:, None])
            dk[:, kvh, :] += scale * (ds.T @ q[rb, h, :])
            dv[:, kvh, :] += p.T @ do[rb, h, :]
            if with_abs:
                w_ = np.abs(ds) + p * bb[h, b0:b0 + len(rb)][:, None]
                adk[:, kvh, :] += scale * (w_.T @ np.abs(q[rb, h, :]))
                adv[:, kvh, :] += p.T @ np.abs(do[rb, h, :])
    return out


def _sees(rows, keys, s_valid, doc, causal):
    """Boolean [len(rows), len(keys)]: key keys[b] is in M(rows[a])."""
    m = np.broadcast_to((keys < s_valid)[None, :], (len(rows), len(keys))).copy()
    if causal:
        m &= keys[None, :] <= rows[:, None]
    if doc is not None:
        m &= doc[keys][None, :] == doc[rows][:, None]
    return m


# ---------------------------------------------------------------------------
# Attention between a query interval and a key interval of one sequence, and
# the merge of partial results. Ring / USP sequence parallelism splits the key
# axis into chunks that visit every rank's queries ("feat(dspark): add Ulysses
# sequence parallel training", Modifications, names ring sequence parallelism
# as the next step; "[trainer] feat: support sequence parallel", review
# overview, builds a (dp, ring, ulysses) mesh); contiguous context parallelism
# gives each rank a contiguous interval of query rows against the whole key
# sequence with causal offsets ("GLM-5.2 131k context parallelism", Purpose:
# contiguous partition mode, q_causal_offsets).
#
# Query row i of the buffer sits at global position q_off + i, key row j at
# k_off + j. Key j is allowed for row i iff j < sk_valid, both positions lie in
# the same document (cu_seqlens over GLOBAL positions) and, when causal,
# k_off + j <= q_off + i. A row with no allowed key has LSE = -inf and O = 0.

def _partial_mask(rows, sk, q_off, k_off, sk_valid, doc, causal):
    gi = q_off + rows
    gj = k_off + np.arange(sk)
    m = np.broadcast_to(np.arange(sk)[None, :] < sk_valid, (len(rows), sk)).copy()
    if causal:
        m &= gj[None, :] <= gi[:, None]
    if doc is not None:
        m &= doc[gj][None, :] == doc[gi][:, None]
    return m


def attn_fwd_partial(q, k, v, scale, q_off=0, k_off=0, sk_valid=None, cu_seqlens=None,
                     causal=True):
    """Partial attention of a query interval against a key interval:
    (O [sq, Hq, d], LSE [Hq, sq]); rows without any allowed key get O = 0 and
    LSE = -inf."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    sq, hq, d = q.shape
    sk, hkv = k.shape[0], k.shape[1]
    g = hq // hkv
    sk_valid = sk if sk_valid is None else sk_valid
    doc = None
    if cu_seqlens is not None:
        doc = doc_of(int(np.asarray(cu_seqlens)[-1]), cu_seqlens)
    o = np.zeros((sq, hq, d))
    lse = np.full((hq, sq), -np.inf)
    for b0 in range(0, sq, ROW_BLOCK):
        rb = np.arange(b0, min(sq, b0 + ROW_BLOCK))
        allowed = _partial_mask(rb, sk, q_off, k_off, sk_valid, doc, causal)
        live = allowed.any(axis=1)
        for h in range(hq):
            z = scale * (q[rb, h, :] @ k[:, h // g, :].T)
            z[~allowed] = -np.inf
            zl = z[live]
            if zl.size == 0:
                continue
            m = zl.max(axis=1)
            lse_b = m + np.log(np.exp(zl - m[:, None]).sum(axis=1))
            p = np.exp(zl - lse_b[:, None])
            o[rb[live], h, :] = p @ v[:, h // g, :]
            lse[h, rb[live]] = lse_b
    return o, lse


def lse_merge(parts):
    """Merge partial results [(O_r, LSE_r), ...] over disjoint key sets:
    LSE = log sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r (rows where
    every LSE_r is -inf stay O = 0, LSE = -inf)."""
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])   # [R, Hq, sq]
    m = lses.max(axis=0)
    msafe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - msafe[None])                                          # [R, Hq, sq]
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, msafe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o = np.zeros_like(np.asarray(parts[0][0], dtype=np.float64))
    for (o_r, _), w_r in zip(parts, w):
        o += np.where(tot > 0, w_r / np.where(tot > 0, tot, 1.0), 0.0).T[:, :, None] * o_r
    return o, lse


def attn_bwd_partial(q, k, v, o, lse, do, scale, q_off=0, k_off=0, sk_valid=None,
                     cu_seqlens=None, causal=True):
    """Backward contributions of one key interval given the FINAL output O and
    the FINAL (merged) LSE of the query rows: (dQ [sq, Hq, d] from these keys
    only, dK and dV [sk, Hkv, d] from these query rows only). Summing dQ over
    the key intervals and dK, dV over the query intervals gives the full
    gradients; D_i = dO_i . O_i uses the final O."""
    q, k, v, o, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    sq, hq, d = q.shape
    sk, hkv = k.shape[0], k.shape[1]
    g = hq // hkv
    sk_valid = sk if sk_valid is None else sk_valid
    doc = None
    if cu_seqlens is not None:
        doc = doc_of(int(np.asarray(cu_seqlens)[-1]), cu_seqlens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b0 in range(0, sq, ROW_BLOCK):
        rb = np.arange(b0, min(sq, b0 + ROW_BLOCK))
        allowed = _partial_mask(rb, sk, q_off, k_off, sk_valid, doc, causal)
        for h in range(hq):
            kvh = h // g
            z = scale * (q[rb, h, :] @ k[:, kvh, :].T)
            lrow = lse[h, rb]
            p = np.where(allowed, np.exp(np.where(allowed, z, 0.0) - np.where(np.isfinite(lrow), lrow, 0.0)[:, None]), 0.0)
            dp = do[rb, h, :] @ v[:, kvh, :].T
            dd = (do[rb, h, :] * o[rb, h, :]).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[rb, h, :] = scale * (ds @ k[:, kvh, :])
            dk[:, kvh, :] += scale * (ds.T @ q[rb, h, :])
            dv[:, kvh, :] += p.T @ do[rb, h, :]
    return dq, dk, dv
