"""CPU bounds check of the GPU kernels' address arithmetic (no GPU needed).

For every shape the GPU tests and the benchmark run, the replica in
tests/kernel_geometry.py evaluates each kernel's load and store offsets for
every workgroup, wave and lane (every tile on small problems, each
workgroup's first and last tile on large ones) and this file checks that
they stay inside the buffers the C ABI is given: the inputs and outputs, and
the workspace layout the library computes (the forward's V copy and split
partials, the backward's D / LSE rows, row-chunk and key-split partials).
The plans (key splits) come from the library's own host queries."""
import numpy as np
import pytest

import workloads
from tests import kernel_geometry as G

BF16 = 0


@pytest.fixture(scope="module")
def L():
    import os

    import ulysses_sequence_parallelism_amd as usp
    if not os.path.exists(usp.LIB_PATH):
        pytest.skip("libusp.so not built")
    return usp.lib()


def within(t, sizes, what):
    for buf, (lo, hi) in t.r.items():
        assert buf in sizes, (what, buf)
        assert lo >= 0 and hi <= sizes[buf], f"{what}: {buf} touches [{lo}, {hi}) of {sizes[buf]}"


def check_fwd(L, m: G.Geom, hq, hkv, d, ws_bytes, out_f32=False, what=""):
    n_split = L.usp_attn_fwd_num_splits(m.s_q, m.q_off, m.s_k, m.k_off, m.s_kv, hq, hkv, d,
                                        int(m.causal), BF16, ws_bytes)
    assert n_split >= 1, what
    g = hq // hkv
    qrows = 32 * (8 // G.hg_for(g))
    st = G.fwd_split_tiles(m, qrows, n_split)
    every = m.s_q * max(m.s_k, 1) <= (1 << 24)
    s_t = G.kmajor_len(m.s_k)
    vcopy = hkv * d * s_t * 2
    t = G.Touch()
    G.kmajor(m.s_k, hkv, d, s_t, t)
    G.fwd(m, hq, hkv, d, n_split, st, every, t, out_f32)
    if n_split > 1:
        G.fwd_merge(m.s_q, hq, d, n_split, t)
        part_bytes = G.align256(n_split * m.s_q * hq * d * 4) + n_split * hq * m.s_q * 4
        assert vcopy + part_bytes <= ws_bytes, what
    assert vcopy <= ws_bytes, what
    sizes = {"q": m.s_q * hq * d, "k_bytes": m.s_k * hkv * d * 2, "v": m.s_k * hkv * d,
             "vt": hkv * d * s_t, "vt_bytes": hkv * d * s_t * 2, "o": m.s_q * hq * d,
             "o32": m.s_q * hq * d, "lse": hq * m.s_q,
             "o_part": n_split * m.s_q * hq * d, "lse_part": n_split * hq * m.s_q}
    within(t, sizes, f"fwd {what}")
    return n_split


def check_bwd(L, m: G.Geom, hq, hkv, d, ws_bytes, what=""):
    n_split = L.usp_attn_bwd_num_splits(m.s_q, m.q_off, m.s_k, m.k_off, m.s_kv, hq, hkv, d,
                                        int(m.causal), BF16, ws_bytes)
    assert n_split >= 1, what
    g = hq // hkv
    qrows = 32 * (4 // G.hg_for(g))
    dq_tiles = G.dq_split_tiles(m, qrows, n_split)
    s_tq = G.kmajor_len(m.s_q)
    every = m.s_q * max(m.s_k, 1) <= (1 << 24)
    rows = G.align256(hq * s_tq * 4) * 2
    t = G.Touch()
    G.rowdot(m.s_q, hq, d, s_tq, t)
    info = G.dkdv(m, hq, hkv, d, s_tq, every, t)
    n_ch = info["n_ch"]
    if n_ch > 1:
        G.dkdv_reduce(m, hkv, d, n_ch, info["cht"], t)
    required = rows + G.align256(2 * n_ch * m.s_k * hkv * d * 4 if n_ch > 1 else 0)
    assert required <= ws_bytes, what
    G.dq(m, hq, hkv, d, s_tq, n_split, dq_tiles, every, t)
    if n_split > 1:
        G.dq_reduce(m, hq, d, n_split, t)
        assert required + n_split * m.s_q * hq * d * 4 <= ws_bytes, what
    sizes = {"q": m.s_q * hq * d, "dout": m.s_q * hq * d, "o": m.s_q * hq * d,
             "q_bytes": m.s_q * hq * d * 2, "dout_bytes": m.s_q * hq * d * 2,
             "k": m.s_k * hkv * d, "v": m.s_k * hkv * d, "k_bytes": m.s_k * hkv * d * 2,
             "v_bytes": m.s_k * hkv * d * 2, "lse": hq * m.s_q, "lse2": hq * s_tq,
             "dd": hq * s_tq, "dq": m.s_q * hq * d, "dk": m.s_k * hkv * d,
             "dv": m.s_k * hkv * d, "part": 2 * n_ch * m.s_k * hkv * d,
             "dq_part": n_split * m.s_q * hq * d}
    within(t, sizes, f"bwd {what}")
    return n_split, n_ch


def full_cases():
    from tests.test_gpu_attention import LONG, SMALL, TILE_COUNTS
    from tests.test_gpu_key_splits import FULL
    out = [(f"tiles_S{s}_{'causal' if c else 'bidir'}", s, s, 4, 1, None, c, 128)
           for s, c, _ in TILE_COUNTS]
    for c in SMALL:
        name, s, s_valid, hq, hkv, cu, causal = c[:7]
        out.append((name, s, s_valid, hq, hkv, cu, causal, c[7] if len(c) > 7 else 128))
    for name, s, s_valid, cu, causal, d, hq, hkv in LONG:
        out.append((name, s, s_valid, hq, hkv, cu, causal, d))
    out += [tuple(c) for c in FULL]
    for name, w in workloads.WORKLOADS.items():
        if w.dtype != "bf16":
            continue
        cu = workloads.cu_seqlens(workloads.doc_lengths(w.s)).tolist() if w.thd else None
        out.append((name, w.s_pad, w.s, w.hq, w.hkv, cu, True, w.d))
    out.append(("bidir_120k", 120000, 120000, 4, 1, None, False, 128))
    return out


@pytest.mark.parametrize("case", full_cases(), ids=lambda c: c[0])
def test_full_sequence_calls_stay_in_bounds(L, case):
    """Forward and backward, with the workspace the queries return (key
    splits where planned) and with the required part alone."""
    name, s, s_valid, hq, hkv, cu, causal, d = case
    m = G.Geom(s_q=s, s_k=s, s_kv=s_valid, cu=cu, causal=causal)
    wf = L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, BF16)
    wb = L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, BF16)
    check_fwd(L, m, hq, hkv, d, wf, what=name)
    check_fwd(L, m, hq, hkv, d, hkv * d * G.kmajor_len(s) * 2, what=name + " (no room)")
    check_bwd(L, m, hq, hkv, d, wb, what=name)
    n_ch = G.dkdv_row_chunks(s, s, hkv)
    req = G.align256(hq * G.kmajor_len(s) * 4) * 2 + \
        G.align256(2 * n_ch * s * hkv * d * 4 if n_ch > 1 else 0)
    assert check_bwd(L, m, hq, hkv, d, req, what=name + " (required)")[0] == 1


def interval_cases():
    from tests.test_gpu_interval import CASES
    out = []
    for c in CASES:
        name, s, s_valid, hq, hkv, qe, ke, cu, causal = c[:9]
        d = c[9] if len(c) > 9 else 128
        for qa, qb in zip(qe[:-1], qe[1:]):
            for ka, kb in zip(ke[:-1], ke[1:]):
                skv = min(max(s_valid - ka, 0), kb - ka)
                out.append((f"{name}[{qa}:{qb}x{ka}:{kb}]", qb - qa, qa, kb - ka, ka, skv, hq,
                            hkv, cu, causal, d))
    # ring of four on the 32K share; USP U2 x R4 at 120K (the last ring rank);
    # the contiguous-CP rank of the benchmark
    s = 32768
    for j in range(4):
        out.append((f"ring32k[{j}]", s, 0, s // 4, j * s // 4, s // 4, 4, 1, None, True, 128))
    s, blk = 120000, 30000
    for j in range(4):
        out.append((f"usp120k[{j}]", blk, 3 * blk, blk, j * blk, blk, 16, 4, None, True, 128))
    out.append(("cp120k_last", 15000, 105000, 120000, 0, 120000, 4, 1, None, True, 128))
    return out


@pytest.mark.parametrize("case", interval_cases(), ids=lambda c: c[0])
def test_interval_calls_stay_in_bounds(L, case):
    name, s_q, q_off, s_k, k_off, s_kv, hq, hkv, cu, causal, d = case
    m = G.Geom(s_q=s_q, s_k=s_k, s_kv=s_kv, q_off=q_off, k_off=k_off, cu=cu, causal=causal)
    wf = L.usp_attn_fwd_workspace_bytes(s_k, hq, hkv, d, BF16)
    wb = L.usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, BF16)
    check_fwd(L, m, hq, hkv, d, wf, out_f32=True, what=name)
    check_bwd(L, m, hq, hkv, d, wb, what=name)


@pytest.mark.parametrize("s_real,p,h,d,es", [
    (120000, 8, 32, 128, 2), (120000, 8, 8, 128, 2), (119999, 8, 32, 128, 2),
    (131072, 2, 32, 128, 2), (512, 2, 8, 64, 4), (999, 3, 6, 2, 2), (1, 8, 8, 4, 4),
    (8192, 8, 8, 64, 2)])
def test_permute_stays_in_bounds(s_real, p, h, d, es):
    for pack in (True, False):
        t = G.Touch()
        cb, s_pad = G.permute(pack, s_real, p, h, d, es, t)
        sizes = {"x": s_real * h * d * es // cb, "y": s_pad * h * d * es // cb}
        within(t, sizes, f"{'pack' if pack else 'unpack'} {s_real} {p} {h} {d}")


@pytest.mark.parametrize("s_q,hq,d", [(30000, 16, 128), (1000, 4, 64), (1, 8, 128)])
def test_merge_stays_in_bounds(s_q, hq, d):
    t = G.Touch()
    G.merge(s_q, hq, d, t)
    n, nl = s_q * hq * d, s_q * hq
    within(t, {"o_a": n, "o_b": n, "o": n, "lse_a": nl, "lse_b": nl, "lse": nl}, "merge")


def test_replica_catches_a_planted_overrun(L):
    """The check is not vacuous: one tile too many in the dK/dV loads, or a
    row clamp removed, reads past the end of Q."""
    m = G.Geom(s_q=1000, s_k=1000, s_kv=1000)
    orig = G.tiles_of

    def one_more(nt, every):
        return orig(np.asarray(nt) + 1, every)

    G.tiles_of = one_more
    try:
        with pytest.raises(AssertionError, match="touches"):
            check_bwd(L, m, 4, 1, 128, L.usp_attn_bwd_workspace_bytes(1000, 4, 1, 128, BF16))
    finally:
        G.tiles_of = orig
