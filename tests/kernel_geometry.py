"""CPU replica of the address arithmetic of libusp's GPU kernels, for bounds
checks without a GPU.

Each function below restates, in numpy, the index formulas one kernel uses
for its global-memory reads and writes (grid decomposition, tile ranges,
key splits and row chunks, the clamped direct loads, the stores), evaluates
them for every workgroup, wave and lane, and returns the touched element or
byte ranges per buffer. tests/test_geometry_cpu.py compares them with the
buffer sizes the C ABI allocates for every shape the tests and the benchmark
use. The formulas are re-typed from the kernel sources (not shared with
them), so a mistake in either shows up as a disagreement.

Tiles: every load offset is a nondecreasing function of the tile's first row
or key (clamps are min(., last) of increasing terms), so for large grids only
each workgroup's first and last tile are evaluated; small problems evaluate
every tile.

C semantics: kernel integer division truncates toward zero (cdiv).
"""
from __future__ import annotations

import dataclasses

import numpy as np

I64 = np.int64


def cdiv(a, b):
    """C integer division (truncation toward zero), elementwise."""
    a = np.asarray(a, dtype=I64)
    q = np.abs(a) // b
    return np.where(a < 0, -q, q)


def hg_for(g):
    return 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1


def kmajor_len(s):
    return (s + 127) // 128 * 128


def align256(x):
    return (x + 255) // 256 * 256


def swz16(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def swz8(r):
    return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1)


def swz_row(d, r):
    return swz16(r) if d == 128 else swz8(r)


@dataclasses.dataclass
class Geom:
    """Mask geometry on global positions (MaskGeom)."""
    s_q: int
    s_k: int
    s_kv: int
    q_off: int = 0
    k_off: int = 0
    cu: list | None = None
    causal: bool = True

    @property
    def lim(self):
        return max(self.q_off + self.s_q, self.k_off + self.s_k)

    def doc_bounds(self, i):
        i = np.asarray(i, dtype=I64)
        if self.cu is None:
            return np.zeros_like(i), np.full_like(i, self.lim)
        cu = np.asarray(self.cu, dtype=I64)
        n = len(cu) - 1
        # largest k in [0, n-1] with cu[k] <= i (k = 0 when none)
        a = np.clip(np.searchsorted(cu[:n], i, side="right") - 1, 0, n - 1)
        lo = np.clip(cu[a], 0, self.lim)
        hi = np.minimum(np.maximum(cu[a + 1], lo), self.lim)
        return lo, hi

    def row_keys(self, r):
        gi = self.q_off + np.asarray(r, dtype=I64)
        blo, bhi = self.doc_bounds(gi)
        lo = np.maximum(blo - self.k_off, 0)
        if self.causal:
            hi = np.minimum(gi - self.k_off, self.s_kv - 1)
        else:
            hi = np.minimum(bhi - self.k_off, self.s_kv) - 1
        return lo, hi

    def key_rows(self, c):
        gj = self.k_off + np.asarray(c, dtype=I64)
        blo, bhi = self.doc_bounds(gj)
        lo = np.maximum(blo, gj if self.causal else 0) - self.q_off
        hi = np.minimum(bhi - self.q_off, self.s_q)
        return lo, hi


class Touch:
    """Collects [lo, hi) element ranges per buffer."""

    def __init__(self):
        self.r = {}

    def add(self, buf, first, last_incl, mask=None):
        first = np.asarray(first, dtype=I64)
        last_incl = np.asarray(last_incl, dtype=I64)
        if mask is not None:
            mask = np.broadcast_to(mask, np.broadcast(first, last_incl).shape)
            first = np.broadcast_to(first, mask.shape)[mask]
            last_incl = np.broadcast_to(last_incl, mask.shape)[mask]
        if first.size == 0:
            return
        lo, hi = int(first.min()), int(last_incl.max()) + 1
        a, b = self.r.get(buf, (lo, hi))
        self.r[buf] = (min(a, lo), max(b, hi))


LANE = np.arange(64, dtype=I64)


def tiles_of(nt, every):
    """Tile indexes evaluated per workgroup: all when `every`, else first and
    last. Returns [n_wg, T] and a validity mask."""
    nt = np.asarray(nt, dtype=I64)
    if every:
        t_max = int(nt.max()) if nt.size else 0
        its = np.broadcast_to(np.arange(max(t_max, 1), dtype=I64), (nt.size, max(t_max, 1)))
    else:
        its = np.stack([np.zeros_like(nt), np.maximum(nt - 1, 0)], axis=1)
    return its, its < nt[:, None]


# ---------------------------------------------------------------------------
# forward (attn_fwd_bf16.hip: fwd_bf16_kernel, split_merge_kernel;
# kmajor.hip: kmajor_kernel)

def fwd_split_tiles(m: Geom, qrows, n_split):
    """split_tiles of the key-split plan (splits.hip): ceil(max tiles / n)."""
    if n_split <= 1:
        return 0
    nqb = -(-m.s_q // qrows)
    last = np.minimum((np.arange(nqb) + 1) * qrows, m.s_q) - 1
    hi = np.minimum(m.q_off + last - m.k_off, m.s_kv - 1) if m.causal else np.full(nqb, m.s_kv - 1)
    nt = np.where(hi >= 0, hi // 64 + 1, 0)
    return int(-(-int(nt.max()) // n_split))


def fwd(m: Geom, hq, hkv, d, n_split, split_tiles, every, t: Touch, out_f32=False):
    BN = 64
    g = hq // hkv
    HG = hg_for(g)
    QROWS = 32 * (8 // HG)
    KC, KK = d // 8, d // 16
    RPP = 64 // KC
    KPW = BN // RPP // 8
    VPW = d // 64
    chunks = g // HG
    n_qblocks = -(-m.s_q // QROWS)
    s_t = kmajor_len(m.s_k)
    bx = np.arange(n_qblocks * n_split, dtype=I64)
    by = np.arange(hkv * chunks, dtype=I64)
    BX, BY = (a.ravel() for a in np.meshgrid(bx, by, indexing="ij"))
    kvh, hc = BY // chunks, BY % chunks
    qb = n_qblocks - 1 - BX // n_split
    zk = BX % n_split
    zs = zk if n_split & 1 else (zk + qb) % n_split
    q0 = qb * QROWS
    q1 = np.minimum(q0 + QROWS, m.s_q)
    kf_lo, kf_hi = m.row_keys(q0)
    kl_lo, kl_hi = m.row_keys(q1 - 1)
    t_split = (cdiv(kf_lo, BN) + zs * split_tiles) * BN
    kmin = np.maximum(kf_lo, t_split) if n_split > 1 else kf_lo
    kmax = np.minimum(kl_hi, t_split + split_tiles * BN - 1) if n_split > 1 else kl_hi
    tstart = cdiv(kmin, BN) * BN
    nt = np.where(kmax >= kmin, cdiv(kmax - tstart, BN) + 1, 0)
    # per wave / lane: Q rows read, O / LSE written
    w = np.arange(8, dtype=I64)
    ln, hl = LANE & 31, LANE >> 5
    wq0 = q0[:, None, None] + (w // HG)[None, :, None] * 32
    qi = wq0 + ln[None, None, :]
    row_ok = qi < m.s_q
    qc = np.where(row_ok, qi, m.s_q - 1)
    head = (kvh * g + hc * HG)[:, None, None] + (w % HG)[None, :, None]
    qe = (qc * hq + head) * d + hl[None, None, :] * 8
    t.add("q", qe, qe + (KK - 1) * 16 + 7)
    has = nt > 0
    live = (has if n_split > 1 else np.ones_like(has))[:, None, None] & row_ok
    oe = (qi * hq + head) * d + hl[None, None, :] * 4
    o_buf = "o_part" if n_split > 1 else ("o32" if out_f32 else "o")
    zso = (zs * m.s_q * hq * d)[:, None, None] if n_split > 1 else 0
    t.add(o_buf, zso + oe, zso + oe + (d // 32 - 1) * 32 + 3 * 8 + 3, live)
    le = head * m.s_q + qi
    zsl = (zs * m.s_q * hq)[:, None, None] if n_split > 1 else 0
    t.add("lse_part" if n_split > 1 else "lse", zsl + le, zsl + le,
          row_ok & (hl[None, None, :] == 0))
    # K and V^T tile loads (bytes), tiles [0, nt)
    its, ok = tiles_of(nt, every)
    t0 = tstart[:, None] + its * BN                                   # [wg, T]
    key_bytes = hkv * d * 2
    q = LANE // KC
    for j in range(KPW):
        part = KPW * w + j                                            # [8]
        first = np.minimum(t0[:, :, None] + RPP * part[None, None, :], m.s_k - 1)
        rel = (np.minimum(t0[:, :, None, None] + RPP * part[None, None, :, None] + q, m.s_k - 1)
               - first[..., None])
        sl = (LANE % KC) ^ swz_row(d, RPP * part[:, None] + q[None, :])
        b = (kvh * d * 2)[:, None, None, None] + first[..., None] * key_bytes + rel * key_bytes \
            + (sl << 4)[None, None]
        t.add("k_bytes", b, b + 15, ok[:, :, None, None])
    vt_row_bytes = s_t * 2
    for j in range(VPW):
        part = VPW * w + j
        base = ((kvh[:, None, None] * d + 8 * part[None, None, :]) * s_t + t0[:, :, None]) * 2
        sl = (LANE & 7) ^ (4 * (part[:, None] & 1) + (LANE[None, :] >> 4))
        off = (LANE >> 3)[None, :] * vt_row_bytes + (sl << 4)
        b = base[..., None] + off[None, None]
        t.add("vt_bytes", b, b + 15, ok[:, :, None, None])
    return dict(s_t=s_t, n_wg=BX.size)


def fwd_merge(s_q, hq, d, nz, t: Touch):
    C = d // 8
    n = s_q * hq * C
    tt = np.arange(n, dtype=I64)
    rh, c = tt // C, tt % C
    i, h = rh // hq, rh % hq
    li = h * s_q + i
    e = rh * d + c * 8
    for z in range(nz):
        t.add("lse_part", z * s_q * hq + li, z * s_q * hq + li)
        t.add("o_part", z * s_q * hq * d + e, z * s_q * hq * d + e + 7)
    t.add("o", e, e + 7)
    t.add("lse", li, li)


def kmajor(s_pad, heads, d, s_t, t: Touch):
    T, KC = 64, d // 8
    bx = np.arange(s_t // T, dtype=I64)
    h = np.arange(heads, dtype=I64)
    BX, H = (a.ravel() for a in np.meshgrid(bx, h, indexing="ij"))
    s0 = BX * T
    tid = np.arange(256, dtype=I64)
    for u in range(T * KC // 256):
        e = tid + 256 * u
        r, c = e // KC, e % KC
        s = s0[:, None] + r[None, :]
        src = (s * heads + H[:, None]) * d + c[None, :] * 8
        t.add("v", src, src + 7, s < s_pad)
    for u in range(d * (T // 8) // 256):
        e = tid + 256 * u
        col, c8 = e >> 3, e & 7
        dst = (H[:, None] * d + col[None, :]) * s_t + s0[:, None] + c8[None, :] * 8
        t.add("vt", dst, dst + 7)


# ---------------------------------------------------------------------------
# backward (attn_bwd_bf16.hip)

def dkdv_row_chunks(s_q, s_k, hkv):
    keys = 128
    items = -(-s_k // keys) * hkv
    tiles = -(-s_q // 64)
    if hkv == 1:
        if items >= 512:
            return 1
        n = min(-(-4096 // items), 16)
    else:
        if items >= 1024:
            return 1
        n = 2
    n = min(n, tiles)
    return n if n > 1 else 1


def rowdot(s_q, hq, d, s_t, t: Touch):
    LPR = d // 8
    n = s_q * hq * LPR
    tt = np.arange(-(-n // 256) * 256, dtype=I64)
    rh, part = tt // LPR, tt % LPR
    live = rh < s_q * hq
    e = rh * d + part * 8
    t.add("o", e, e + 7, live)
    t.add("dout", e, e + 7, live)
    i, h = rh // hq, rh % hq
    wr = live & (part == 0)
    t.add("dd", h * s_t + i, h * s_t + i, wr)
    t.add("lse2", h * s_t + i, h * s_t + i, wr)
    t.add("lse", h * s_q + i, h * s_q + i, wr)


def dkdv(m: Geom, hq, hkv, d, s_tq, every, t: Touch):
    BQ, KG = 64, 4
    KEYS = 32 * KG
    KC, KK, DB = d // 8, d // 16, d // 32
    RPP = 64 // KC
    g = hq // hkv
    n_kb = -(-m.s_k // KEYS)
    n_ch = dkdv_row_chunks(m.s_q, m.s_k, hkv)
    tiles = -(-m.s_q // BQ)
    cht = -(-tiles // n_ch)
    bx = np.arange(n_kb * n_ch, dtype=I64)
    kv = np.arange(hkv, dtype=I64)
    BX, KVH = (a.ravel() for a in np.meshgrid(bx, kv, indexing="ij"))
    cch, kbi = BX // n_kb, BX % n_kb
    j0 = kbi * KEYS
    j1 = np.minimum(j0 + KEYS, m.s_k)
    w = np.arange(8, dtype=I64)
    grp, role = w % KG, w // KG
    ln, hl = LANE & 31, LANE >> 5
    key = j0[:, None, None] + grp[None, :, None] * 32 + ln[None, None, :]
    kc = np.minimum(key, m.s_k - 1)
    # stationary K / V fragments
    se = (kc * hkv + KVH[:, None, None]) * d + hl * 8
    t.add("k", se, se + (KK - 1) * 16 + 7, role[None, :, None] == 0)
    t.add("v", se, se + (KK - 1) * 16 + 7, role[None, :, None] == 1)
    rf_lo, rf_hi = m.key_rows(j0)
    rl_lo, rl_hi = m.key_rows(j1 - 1)
    rstart = np.maximum(rf_lo, 0)
    rend = rl_hi - 1
    tstart = cdiv(rstart, BQ) * BQ
    tlast = (m.s_q - 1) // BQ
    clo = np.maximum(cdiv(tstart, BQ), tlast - (cch + 1) * cht + 1)
    chi = np.minimum(cdiv(rend, BQ), tlast - cch * cht)
    ntr = np.where((j0 < m.s_kv) & (rend >= rstart) & (chi >= clo), chi - clo + 1, 0)
    nt = ntr * g
    stores = (ntr > 0) if n_ch > 1 else np.ones_like(ntr, dtype=bool)
    # stores of dV (role 0) and dK (role 1), or of this chunk's partials
    oe = (key * hkv + KVH[:, None, None]) * d + hl * 4
    last = (DB - 1) * 32 + 3 * 8 + 3
    live = (key < m.s_k) & stores[:, None, None]
    if n_ch > 1:
        slice_ = m.s_k * hkv * d
        base = (role[None, :, None] * n_ch + cch[:, None, None]) * slice_
        t.add("part", base + oe, base + oe + last, live)
    else:
        t.add("dv", oe, oe + last, live & (role[None, :, None] == 0))
        t.add("dk", oe, oe + last, live & (role[None, :, None] == 1))
    # tile loads by the four loading waves: Q / dO rows, LSE / D values
    its, ok = tiles_of(nt, every)
    ok = ok & stores[:, None]
    r0 = (chi[:, None] - its // g) * BQ
    h = KVH[:, None] * g + its % g
    row_bytes = hq * d * 2
    HALF, PARTS = KG // 2, BQ // RPP // (KG // 2)
    q = LANE // KC
    for r1 in range(KG):
        p0 = (r1 % HALF) * PARTS
        buf = "q_bytes" if r1 < HALF else "dout_bytes"
        base = h * (d * 2)
        for pp in range(PARTS):
            part = p0 + pp
            full = r0 + BQ <= m.s_q
            first = np.where(full, r0 + RPP * part, np.minimum(r0 + RPP * part, m.s_q - 1))
            rel = np.where(full[..., None], q,
                           np.minimum(r0[..., None] + RPP * part + q, m.s_q - 1) - first[..., None])
            sl = (LANE % KC) ^ swz_row(d, RPP * part + q)
            b = base[..., None] + first[..., None] * row_bytes + rel * row_bytes + (sl << 4)
            t.add(buf, b, b + 15, ok[..., None])
        if r1 % HALF == 0:
            i0 = np.minimum(r0, m.s_q - 1)
            rel = np.minimum(r0[..., None] + LANE, m.s_q - 1) - i0[..., None]
            e = h[..., None] * s_tq + i0[..., None] + rel
            t.add("lse2" if r1 == 0 else "dd", e, e, ok[..., None])
    return dict(n_ch=n_ch, cht=cht, n_kb=n_kb)


def dkdv_reduce(m: Geom, hkv, d, n_ch, cht, t: Touch):
    n4 = m.s_k * hkv * d // 4
    i = np.arange(2 * n4, dtype=I64)
    tt = (i >= n4).astype(I64)
    e = i - tt * n4
    for c in range(n_ch):
        src = (tt * n_ch * n4 + e + c * n4) * 4
        t.add("part", src, src + 3)
    t.add("dv", e * 4, e * 4 + 3, tt == 0)
    t.add("dk", e * 4, e * 4 + 3, tt == 1)


def dq_split_tiles(m: Geom, qrows, n_split):
    if n_split <= 1:
        return 0
    nqb = -(-m.s_q // qrows)
    last = np.minimum((np.arange(nqb) + 1) * qrows, m.s_q) - 1
    hi = np.minimum(m.q_off + last - m.k_off, m.s_kv - 1) if m.causal else np.full(nqb, m.s_kv - 1)
    nt = np.where(hi >= 0, hi // 32 + 1, 0)
    return int(-(-int(nt.max()) // n_split))


def dq(m: Geom, hq, hkv, d, s_tq, dq_split, dq_tiles, every, t: Touch):
    BN = 32
    g = hq // hkv
    HG = hg_for(g)
    QROWS = 32 * (4 // HG)
    KC, KK, DB = d // 8, d // 16, d // 32
    RPP = 64 // KC
    PPW = BN // RPP // 4
    chunks = g // HG
    n_blocks = -(-m.s_q // QROWS)
    bx = np.arange(n_blocks * dq_split, dtype=I64)
    by = np.arange(hkv * chunks, dtype=I64)
    BX, BY = (a.ravel() for a in np.meshgrid(bx, by, indexing="ij"))
    kvh, hc = BY // chunks, BY % chunks
    qb = n_blocks - 1 - BX // dq_split
    zk = BX % dq_split
    zs = zk if dq_split & 1 else (zk + qb) % dq_split
    q0 = qb * QROWS
    q1 = np.minimum(q0 + QROWS, m.s_q)
    w = np.arange(4, dtype=I64)
    ln, hl = LANE & 31, LANE >> 5
    qi = q0[:, None, None] + (w // HG)[None, :, None] * 32 + ln
    row_ok = qi < m.s_q
    qc = np.where(row_ok, qi, m.s_q - 1)
    head = (kvh * g + hc * HG)[:, None, None] + (w % HG)[None, :, None]
    kf_lo, _ = m.row_keys(q0)
    _, kl_hi = m.row_keys(q1 - 1)
    t_split = (cdiv(kf_lo, BN) + zs * dq_tiles) * BN
    kmin = np.maximum(kf_lo, t_split) if dq_split > 1 else kf_lo
    kmax = np.minimum(kl_hi, t_split + dq_tiles * BN - 1) if dq_split > 1 else kl_hi
    tstart = cdiv(kmin, BN) * BN
    nt = np.where(kmax >= kmin, cdiv(kmax - tstart, BN) + 1, 0)
    run = (nt > 0) if dq_split > 1 else np.ones_like(nt, dtype=bool)
    rr = run[:, None, None]
    e = (qc * hq + head) * d + hl * 8
    t.add("q", e, e + (KK - 1) * 16 + 7, rr)
    t.add("dout", e, e + (KK - 1) * 16 + 7, rr)
    t.add("lse", head * m.s_q + qc, head * m.s_q + qc, rr)
    t.add("dd", head * s_tq + qc, head * s_tq + qc, rr)
    oe = (qi * hq + head) * d + hl * 4
    last = (DB - 1) * 32 + 3 * 8 + 3
    if dq_split > 1:
        zo = (zs * m.s_q * hq * d)[:, None, None]
        t.add("dq_part", zo + oe, zo + oe + last, rr & row_ok)
    else:
        t.add("dq", oe, oe + last, row_ok)
    its, ok = tiles_of(nt, every)
    t0 = tstart[:, None] + its * BN
    key_bytes = hkv * d * 2
    q = LANE // KC
    for j in range(PPW):
        part = PPW * w + j
        first = np.minimum(t0[:, :, None] + RPP * part, m.s_k - 1)
        rel = np.minimum(t0[:, :, None, None] + RPP * part[:, None] + q, m.s_k - 1) - first[..., None]
        sl = (LANE % KC) ^ swz_row(d, RPP * part[:, None] + q)
        b = (kvh * d * 2)[:, None, None, None] + first[..., None] * key_bytes + rel * key_bytes + \
            (sl << 4)[None, None]
        t.add("k_bytes", b, b + 15, (ok & run[:, None])[:, :, None, None])
        t.add("v_bytes", b, b + 15, (ok & run[:, None])[:, :, None, None])
    return dict(n_blocks=n_blocks)


def dq_reduce(m: Geom, hq, d, nz, t: Touch):
    n4 = m.s_q * hq * d // 4
    i = np.arange(n4, dtype=I64)
    stride4 = m.s_q * hq * d // 4
    for z in range(nz):
        t.add("dq_part", (i + z * stride4) * 4, (i + z * stride4) * 4 + 3)
    t.add("dq", i * 4, i * 4 + 3)


# ---------------------------------------------------------------------------
# layout transform (permute.hip) and ring merge (merge.hip)

def permute(pack, s_real, p, h, d, es, t: Touch):
    """Chunk indexes of permute_kernel: returns element ranges in units of the
    kernel's chunk (the widest of 16, 8, 4 bytes dividing a run)."""
    row_bytes = h * d * es
    run_bytes = row_bytes // p
    cb = 16 if run_bytes % 16 == 0 else 8 if run_bytes % 8 == 0 else 4
    s_pad = p * (-(-s_real // p))
    row_chunks, run_chunks = row_bytes // cb, run_bytes // cb
    rows = s_pad if pack else s_real
    total = rows * row_chunks
    tt = np.arange(total, dtype=I64)
    s = tt // row_chunks
    c = tt - s * row_chunks
    r = c // run_chunks
    off = c - r * run_chunks
    y = (r * s_pad + s) * run_chunks + off
    if pack:
        t.add("x", tt, tt, s < s_real)
        t.add("y", y, y)
    else:
        t.add("y", y, y)
        t.add("x", tt, tt)
    return cb, s_pad


def merge(s_q, hq, d, t: Touch):
    C = d // 4
    n = s_q * hq * C
    tt = np.arange(n, dtype=I64)
    rh, c = tt // C, tt % C
    i, h = rh // hq, rh % hq
    li = h * s_q + i
    e = rh * d + c * 4
    for b in ("o_a", "o_b", "o"):
        t.add(b, e, e + 3)
    for b in ("lse_a", "lse_b", "lse"):
        t.add(b, li, li)


# ---------------------------------------------------------------------------
# longest-first block order of calls with documents (splits.hip)

def block_costs(m: Geom, kind, n, block, tile):
    """Tiles each block walks: kind 0, query blocks of `block` rows over key
    tiles of `tile`; kind 1, key blocks of `block` keys over row tiles of
    `tile` (as block_cost_kernel)."""
    b = np.arange(n, dtype=I64)
    if kind == 0:
        q0 = b * block
        q1 = np.minimum(q0 + block, m.s_q)
        lo, _ = m.row_keys(q0)
        _, hi = m.row_keys(q1 - 1)
        t0 = cdiv(lo, tile) * tile
        return np.where(hi >= lo, cdiv(hi - t0, tile) + 1, 0)
    j0 = b * block
    j1 = np.minimum(j0 + block, m.s_k)
    rf_lo, _ = m.key_rows(j0)
    _, rl_hi = m.key_rows(j1 - 1)
    rstart = np.maximum(rf_lo, 0)
    rend = rl_hi - 1
    return np.where((j0 < m.s_kv) & (rend >= rstart), cdiv(rend, tile) - cdiv(rstart, tile) + 1, 0)


def longest_first(cost):
    """Block indexes by decreasing cost, ties by index."""
    cost = np.asarray(cost)
    return np.lexsort((np.arange(len(cost)), -cost))
