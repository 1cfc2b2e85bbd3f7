"""CPU-side checks of the C ABI: the library loads, exports every entry point
include/usp.h declares, and rejects bad arguments on the host before any HIP
call (so these run without a GPU; no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "usp.h")

OK, INVALID, UNSUPPORTED, NULLP, HIPERR, WORKSPACE = 0, -1, -2, -3, -4, -5
BF16, FP32 = 0, 1


@pytest.fixture(scope="module")
def L():
    import ulysses_sequence_parallelism_amd as usp
    if not os.path.exists(usp.LIB_PATH):
        pytest.skip("libusp.so not built")
    return usp.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(usp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_hot_path_calls():
    names = declared_functions()
    for n in ("usp_pad_pack_seq2head", "usp_attn_fwd", "usp_attn_bwd", "usp_unpack_head2seq"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    import ulysses_sequence_parallelism_amd as usp
    out = subprocess.run(["nm", "-D", "--defined-only", usp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (usp_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    # and the Python binding has a function of the same name
    for name in declared_functions():
        assert callable(getattr(usp, name)), name


def test_version_and_status_strings(L):
    assert L.usp_version() == 121
    for s in (OK, INVALID, UNSUPPORTED, NULLP, HIPERR, WORKSPACE, 12345):
        assert isinstance(L.usp_status_string(s), bytes)
    assert L.usp_status_string(0) == b"ok"


def test_buffer_checks_toggle(L):
    """usp_check_buffers sets the optional buffer checks and returns the
    previous state; a negative argument only reads it."""
    start = L.usp_check_buffers(-1)
    assert start in (0, 1)
    try:
        assert L.usp_check_buffers(1) == start
        assert L.usp_check_buffers(-1) == 1
        assert L.usp_check_buffers(0) == 1
        assert L.usp_check_buffers(-1) == 0
    finally:
        L.usp_check_buffers(start)


def test_padded_len_matches_oracle(L):
    for s in list(range(0, 40)) + [119999, 120000, 131071]:
        for p in (1, 2, 3, 4, 8):
            assert L.usp_padded_len(s, p) == oracle.padded_len(s, p)
    assert L.usp_padded_len(5, 0) == -1
    assert L.usp_padded_len(-1, 2) == -1


A = 1 << 20  # fake, 16-byte-aligned addresses: never dereferenced by a rejected call
B = 1 << 40


def pack(L, x, y, s, p, h, d, dt):
    return L.usp_pad_pack_seq2head(ctypes.c_void_p(x), ctypes.c_void_p(y), s, p, h, d, dt, None)


def unpack(L, y, x, s, p, h, d, dt):
    return L.usp_unpack_head2seq(ctypes.c_void_p(y), ctypes.c_void_p(x), s, p, h, d, dt, None)


def test_permute_argument_errors(L):
    for f in (pack, unpack):
        assert f(L, A, B, 16, 3, 8, 128, BF16) == INVALID       # heads not divisible
        assert f(L, A, B, 16, 0, 8, 128, BF16) == INVALID       # p < 1
        assert f(L, A, B, -1, 2, 8, 128, BF16) == INVALID       # s < 0
        assert f(L, A, B, 16, 2, 8, 0, BF16) == INVALID         # d < 1
        assert f(L, A, B, 16, 2, 8, 128, 7) == UNSUPPORTED      # dtype
        assert f(L, A, B, 16, 2, 2, 1, BF16) == UNSUPPORTED     # 2-byte runs
        assert f(L, A + 8, B, 16, 2, 8, 128, BF16) == INVALID   # misaligned
        assert f(L, A, B + 4, 16, 2, 8, 128, BF16) == INVALID
        assert f(L, 0, B, 16, 2, 8, 128, BF16) == NULLP
        assert f(L, A, 0, 16, 2, 8, 128, BF16) == NULLP
        assert f(L, A, A + 4096, 16, 2, 8, 128, BF16) == INVALID  # overlap
        assert f(L, A, B, 0, 2, 8, 128, BF16) == OK             # nothing to do, no HIP call
        assert f(L, 0, 0, 0, 2, 8, 128, FP32) == OK


def fwd(L, s_pad=256, s_valid=256, cu=None, n_docs=0, hq=4, hkv=1, d=128, scale=0.088, causal=1,
        dt=BF16, ws=3 << 30, ws_bytes=1 << 30, ptrs=None):
    q, k, v, o, lse = ptrs or (A, A + (1 << 24), A + (2 << 24), A + (3 << 24), A + (4 << 24))
    return L.usp_attn_fwd(*(ctypes.c_void_p(x) for x in (q, k, v, o, lse, ws)), ws_bytes, s_pad,
                          s_valid, ctypes.c_void_p(cu), n_docs, hq, hkv, d, scale, causal, dt,
                          None)


def bwd(L, s_pad=256, s_valid=256, cu=None, n_docs=0, hq=4, hkv=1, d=128, scale=0.088, causal=1,
        dt=BF16, ws=3 << 30, ws_bytes=1 << 30, ptrs=None):
    base = [A + (i << 24) for i in range(9)]
    ptrs = ptrs or base
    return L.usp_attn_bwd(*(ctypes.c_void_p(x) for x in ptrs), ctypes.c_void_p(ws), ws_bytes,
                          s_pad, s_valid, ctypes.c_void_p(cu), n_docs, hq, hkv, d, scale, causal,
                          dt, None)


@pytest.mark.parametrize("f", [fwd, bwd])
def test_attention_argument_errors(L, f):
    assert f(L, hq=6, hkv=4) == INVALID                 # hq % hkv
    assert f(L, s_valid=0) == INVALID
    assert f(L, s_valid=257) == INVALID
    assert f(L, s_pad=0, s_valid=0) == INVALID
    assert f(L, cu=A + (8 << 24), n_docs=2, s_valid=250) == INVALID  # packed docs + padding
    assert f(L, cu=A + (8 << 24), n_docs=0) == INVALID
    assert f(L, cu=A + (8 << 24) + 2, n_docs=2) == INVALID            # misaligned offsets
    assert f(L, d=96) == UNSUPPORTED                    # head dims 64 and 128 are built
    assert f(L, d=32) == UNSUPPORTED
    assert f(L, d=96, dt=FP32) == UNSUPPORTED
    assert f(L, dt=3) == UNSUPPORTED
    assert f(L, scale=0.0) == INVALID
    assert f(L, scale=float("nan")) == INVALID
    assert f(L, causal=2) == INVALID
    assert f(L, ws=0) == WORKSPACE
    assert f(L, ws_bytes=16) == WORKSPACE
    assert f(L, ws=(3 << 30) + 8) == INVALID            # misaligned workspace
    if f is fwd:  # the forward needs its V copy (128 x 256 x 2 bytes) at least
        assert f(L, ws_bytes=128 * 256 * 2 - 16) == WORKSPACE
    else:  # the backward its D and LSE rows (two 4 x 256 fp32 arrays) and chunk partials
        req = L.usp_attn_bwd_workspace_bytes(256, 4, 1, 128, BF16) - dq_room(256, 4, 1, 128)
        assert f(L, ws_bytes=req - 16) == WORKSPACE


def test_attention_null_and_alias(L):
    z = [A + (i << 24) for i in range(9)]
    assert fwd(L, ptrs=(0, z[1], z[2], z[3], z[4])) == NULLP
    assert fwd(L, ptrs=(z[0], z[1], z[2], z[0] + 1024, z[4])) == INVALID  # o overlaps q
    assert fwd(L, ptrs=(z[0], z[1], z[2], z[3], z[3] + 64)) == INVALID    # lse overlaps o
    assert fwd(L, ws=z[0]) == INVALID                                     # workspace overlaps q
    p = list(z)
    p[6] = p[0]  # dq aliases q
    assert bwd(L, ptrs=p) == INVALID
    p = list(z)
    p[8] = p[7]  # dv aliases dk
    assert bwd(L, ptrs=p) == INVALID
    p = list(z)
    p[5] = 0
    assert bwd(L, ptrs=p) == NULLP


def fwd_iv(L, s_q=200, q_off=0, s_k=256, k_off=0, s_kv=256, cu=None, n_docs=0, hq=4, hkv=1,
           d=128, scale=0.088, causal=1, dt=BF16, odt=FP32, ws=3 << 30, ws_bytes=1 << 30,
           ptrs=None):
    q, k, v, o, lse = ptrs or (A, A + (1 << 24), A + (2 << 24), A + (3 << 24), A + (4 << 24))
    return L.usp_attn_fwd_interval(*(ctypes.c_void_p(x) for x in (q, k, v, o, lse, ws)), ws_bytes,
                                   s_q, q_off, s_k, k_off, s_kv, ctypes.c_void_p(cu), n_docs, hq,
                                   hkv, d, scale, causal, dt, odt, None)


def bwd_iv(L, s_q=200, q_off=0, s_k=256, k_off=0, s_kv=256, cu=None, n_docs=0, hq=4, hkv=1,
           d=128, scale=0.088, causal=1, dt=BF16, gdt=FP32, acc=1, ws=3 << 30,
           ws_bytes=1 << 30, ptrs=None):
    ptrs = ptrs or [A + (i << 24) for i in range(9)]
    return L.usp_attn_bwd_interval(*(ctypes.c_void_p(x) for x in ptrs), ctypes.c_void_p(ws),
                                   ws_bytes, s_q, q_off, s_k, k_off, s_kv, ctypes.c_void_p(cu),
                                   n_docs, hq, hkv, d, scale, causal, dt, gdt, acc, None)


@pytest.mark.parametrize("f", [fwd_iv, bwd_iv])
def test_interval_argument_errors(L, f):
    assert f(L, s_q=0) == INVALID
    assert f(L, s_k=0, s_kv=0) == INVALID
    assert f(L, q_off=-1) == INVALID
    assert f(L, k_off=-5) == INVALID
    assert f(L, q_off=(1 << 30) - 100) == INVALID       # global positions are 32-bit
    assert f(L, k_off=(1 << 30) - 100) == INVALID
    assert f(L, s_kv=-1) == INVALID
    assert f(L, s_kv=257) == INVALID
    assert f(L, hq=6, hkv=4) == INVALID
    assert f(L, cu=A + (8 << 24), n_docs=0) == INVALID
    assert f(L, cu=A + (8 << 24) + 2, n_docs=2) == INVALID
    assert f(L, d=96) == UNSUPPORTED
    assert f(L, dt=3) == UNSUPPORTED
    assert f(L, scale=-1.0) == INVALID
    assert f(L, causal=-1) == INVALID
    assert f(L, ws=0) == WORKSPACE
    assert f(L, ws_bytes=16) == WORKSPACE


def test_interval_output_dtype_and_accumulate_errors(L):
    assert fwd_iv(L, odt=5) == UNSUPPORTED
    assert fwd_iv(L, dt=FP32, d=64, odt=BF16) == UNSUPPORTED   # fp32 inputs give fp32 O
    assert bwd_iv(L, gdt=5) == UNSUPPORTED
    assert bwd_iv(L, dt=FP32, d=64, gdt=BF16, acc=0) == UNSUPPORTED
    assert bwd_iv(L, gdt=BF16, acc=1) == INVALID              # accumulation is fp32 only
    assert bwd_iv(L, acc=2) == INVALID
    z = [A + (i << 24) for i in range(9)]
    assert fwd_iv(L, ptrs=(z[0], z[1], z[2], z[1] + 256, z[4])) == INVALID  # o overlaps k
    p = list(z)
    p[7] = p[6] + 4096  # dk overlaps dq
    assert bwd_iv(L, ptrs=p) == INVALID


def merge(L, oa=A, la=A + (1 << 24), ob=A + (2 << 24), lb=A + (3 << 24), o=A + (4 << 24),
          lse=A + (5 << 24), s_q=100, hq=4, d=128, odt=FP32):
    return L.usp_attn_merge(*(ctypes.c_void_p(x) for x in (oa, la, ob, lb, o, lse)), s_q, hq, d,
                            odt, None)


def test_merge_argument_errors(L):
    assert merge(L, s_q=0) == INVALID
    assert merge(L, hq=0) == INVALID
    assert merge(L, s_q=1 << 22, hq=8, d=128) == INVALID     # 32-bit element count
    assert merge(L, d=96) == UNSUPPORTED
    assert merge(L, odt=4) == UNSUPPORTED
    assert merge(L, oa=0) == NULLP
    assert merge(L, lse=0) == NULLP
    assert merge(L, o=A + (4 << 24) + 4) == INVALID          # misaligned
    assert merge(L, o=A + 1024) == INVALID                    # partly overlaps o_a
    assert merge(L, o=A, odt=BF16) == INVALID                 # in place needs fp32 O
    assert merge(L, lse=A + (1 << 24) + 16) == INVALID        # partly overlaps lse_a
    assert merge(L, o=A + (1 << 24)) == INVALID               # O over lse_a


def dkdv_chunks(s_q, s_k, hkv):
    """Row chunks per key block of the bf16 dK/dV kernel. One KV head: 1 when
    the 128-key blocks number at least 512, else enough for about 4096 (block,
    chunk) items, at most 16. Several KV heads: 1 from 1024 (block, head)
    items, else 2. Never more than the number of 64-row tiles."""
    items = -(-s_k // 128) * hkv
    if hkv == 1:
        if items >= 512:
            return 1
        n = min(-(-4096 // items), 16)
    else:
        if items >= 1024:
            return 1
        n = 2
    return max(1, min(n, -(-s_q // 64)))


def dq_split_cap(s_q, hq, hkv):
    """Most dQ key splits: 1 when the dQ grid (workgroups of HG query heads x
    4/HG blocks of 32 rows) has 1024 workgroups or more, else enough for
    about 2048, at most 8."""
    g = hq // hkv
    hg = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    wgs = -(-s_q // (32 * (4 // hg))) * hkv * (g // hg)
    return 1 if wgs >= 1024 else min(8, -(-2048 // wgs))


def order_bytes(n):
    """A block order table of n blocks: costs, ranks, then the order (int32
    each, 256-byte aligned)."""
    return 3 * (-(-n * 4 // 256) * 256)


def dq_room(s_q, hq, hkv, d, s_k=None):
    """Room the backward workspace query adds beyond the required part: the dQ
    key-split partials, or the two block orders of a call with documents (dK/dV
    key blocks of 128, dQ query blocks of 32 (4 / HG) rows), whichever is
    larger (the two are never used together)."""
    s_k = s_q if s_k is None else s_k
    z = dq_split_cap(s_q, hq, hkv)
    g = hq // hkv
    hg = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    orders = order_bytes(-(-s_k // 128)) + order_bytes(-(-s_q // (32 * (4 // hg))))
    return max(z * s_q * hq * d * 4 if z > 1 else 0, orders)


def test_workspace_sizes(L):
    for s in (1, 100, 128, 129, 120000, 131072):
        f = L.usp_attn_fwd_workspace_bytes(s, 4, 1, 128, BF16)
        b = L.usp_attn_bwd_workspace_bytes(s, 4, 1, 128, BF16) - dq_room(s, 4, 1, 128)
        assert f >= 128 * s * 2 and f % 16 == 0
        # fp32 partial dK and dV per row chunk when the rows are split
        n = dkdv_chunks(s, s, 1)
        part = 2 * n * s * 128 * 4 if n > 1 else 0
        # D and LSE * log2(e) per (head, row), fp32
        assert 2 * 4 * s * 4 <= b - part < 2 * 4 * (s + 128) * 4 + 512
    assert dkdv_chunks(120000, 120000, 1) == 1 and dkdv_chunks(8192, 8192, 1) == 16
    assert dkdv_chunks(32768, 32768, 1) == 16 and dkdv_chunks(100, 100, 1) == 2
    assert dkdv_chunks(8192, 8192, 8) == 2 and dkdv_chunks(8192, 8192, 16) == 1
    assert L.usp_attn_fwd_workspace_bytes(512, 4, 2, 64, FP32) == 0
    assert L.usp_attn_bwd_workspace_bytes(512, 4, 2, 64, FP32) == 512 * 4 * 4
    assert L.usp_attn_fwd_workspace_bytes(0, 4, 1, 128, BF16) == 0
    # interval: the query rows and, through the row chunks, the keys
    for s_q, s_k in ((100, 1000), (1000, 100), (512, 512), (30000, 30000)):
        for hkv, d in ((1, 128), (4, 64)):
            b = L.usp_attn_bwd_interval_workspace_bytes(s_q, s_k, 4 * hkv, hkv, d, BF16)
            b -= dq_room(s_q, 4 * hkv, hkv, d, s_k)
            n = dkdv_chunks(s_q, s_k, hkv)
            part = 2 * n * s_k * hkv * d * 4 if n > 1 else 0
            assert 2 * 4 * hkv * s_q * 4 <= b - part < 2 * 4 * hkv * (s_q + 128) * 4 + 512
    assert L.usp_attn_bwd_interval_workspace_bytes(512, 512, 4, 1, 128, BF16) == \
        L.usp_attn_bwd_workspace_bytes(512, 4, 1, 128, BF16)
    assert L.usp_attn_bwd_interval_workspace_bytes(300, 700, 4, 2, 64, FP32) == 300 * 4 * 4


def fwd_split_cap(s, hq, hkv):
    """Most key splits the bf16 forward may run for s query rows: 1 when the
    unsplit grid (workgroups of HG query heads x 8/HG blocks of 32 rows) has
    512 workgroups or more, else enough for about 1024, at most 8."""
    g = hq // hkv
    hg = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    wgs = -(-s // (32 * (8 // hg))) * hkv * (g // hg)
    return 1 if wgs >= 512 else min(8, -(-1024 // wgs))


def test_fwd_workspace_and_key_splits(L):
    vcopy = lambda s, hkv, d: hkv * d * ((s + 127) // 128 * 128) * 2
    for s, hq, hkv, d in ((8192, 4, 1, 128), (16384, 4, 1, 128), (16385, 4, 1, 128),
                          (32768, 4, 1, 128), (1000, 8, 2, 64), (120000, 4, 1, 128),
                          (131072, 16, 4, 128), (64, 4, 1, 128)):
        z = fwd_split_cap(s, hq, hkv)
        # fp32 partial O (256-byte aligned) and LSE per split, or the block
        # order of a call with documents (query blocks of 32 (8 / HG) rows),
        # whichever is larger
        room = (-(-z * s * hq * d * 4 // 256) * 256 + z * hq * s * 4) if z > 1 else 0
        g = hq // hkv
        hg = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
        room = max(room, order_bytes(-(-s // (32 * (8 // hg)))))
        ws = L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, BF16)
        assert ws == vcopy(s, hkv, d) + room
        for causal in (0, 1):
            n = L.usp_attn_fwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, BF16, ws)
            assert 1 <= n <= z
            # deterministic, and one pass without room for the partials
            assert n == L.usp_attn_fwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, BF16, ws)
            assert L.usp_attn_fwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, BF16,
                                             vcopy(s, hkv, d)) == 1
            assert L.usp_attn_fwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, FP32, ws) == 1
    split = lambda *a: L.usp_attn_fwd_num_splits(*a, L.usp_attn_fwd_workspace_bytes(
        a[2], a[5], a[6], a[7], BF16))
    # the short causal share (128 workgroups, a 128-tile triangle) is split; the
    # long ones, and the contiguous context-parallel rank, run one pass
    assert split(8192, 0, 8192, 0, 8192, 4, 1, 128, 1, BF16) > 1
    assert split(16384, 0, 16384, 0, 16384, 4, 1, 128, 1, BF16) > 1
    for s in (32768, 120000):
        assert split(s, 0, s, 0, s, 4, 1, 128, 1, BF16) == 1
    assert split(15000, 105000, 120000, 0, 120000, 4, 1, 128, 1, BF16) == 1
    # fewer than 8 tiles per split: one pass
    assert split(300, 0, 300, 0, 300, 4, 1, 128, 1, BF16) == 1
    # dQ: the same for the backward's workspace and its dQ key splits
    for s, hq, hkv, d in ((8192, 4, 1, 128), (16384, 4, 1, 128), (32768, 4, 1, 128),
                          (1000, 8, 2, 64), (120000, 4, 1, 128), (64, 4, 1, 128)):
        wb = L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, BF16)
        req = wb - dq_room(s, hq, hkv, d)
        for causal in (0, 1):
            n = L.usp_attn_bwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, BF16, wb)
            assert 1 <= n <= dq_split_cap(s, hq, hkv)
            assert L.usp_attn_bwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, BF16, req) == 1
            assert L.usp_attn_bwd_num_splits(s, 0, s, 0, s, hq, hkv, d, causal, FP32, wb) == 1
    bsplit = lambda s, hq, hkv, d: L.usp_attn_bwd_num_splits(
        s, 0, s, 0, s, hq, hkv, d, 1, BF16, L.usp_attn_bwd_workspace_bytes(s, hq, hkv, d, BF16))
    assert bsplit(8192, 4, 1, 128) > 1 and bsplit(16384, 4, 1, 128) > 1
    assert bsplit(32768, 4, 1, 128) == 1 and bsplit(120000, 4, 1, 128) == 1
    assert L.usp_attn_bwd_num_splits(0, 0, 8, 0, 8, 4, 1, 128, 1, BF16, 1 << 30) == -1
    # argument errors as in the interval forward
    assert L.usp_attn_fwd_num_splits(0, 0, 8, 0, 8, 4, 1, 128, 1, BF16, 1 << 30) == -1
    assert L.usp_attn_fwd_num_splits(8, 0, 8, 0, 8, 4, 1, 96, 1, BF16, 1 << 30) == -2
    assert L.usp_attn_fwd_num_splits(8, 0, 8, 0, 9, 4, 1, 128, 1, BF16, 1 << 30) == -1


def test_key_split_plans_fit_the_workspace(L):
    """Whatever workspace a caller passes (at least the required part), the
    planned splits' partials fit inside it: forward O + LSE per split after
    the V copy, dQ per split after the backward's required part. Swept over
    interval shapes (more rows than keys, offsets), masks, head layouts and
    workspace sizes from the minimum to the query's size and beyond."""
    import itertools
    vcopy = lambda s_k, hkv, d: hkv * d * ((s_k + 127) // 128 * 128) * 2
    shapes = [(8192, 0, 8192, 0), (3000, 0, 1000, 500), (1500, 2000, 3500, 0), (700, 0, 5000, 0),
              (16384, 0, 16384, 0), (4096, 4096, 4096, 0), (100, 0, 100, 0)]
    for (s_q, q_off, s_k, k_off), (hq, hkv, d), causal in itertools.product(
            shapes, ((4, 1, 128), (16, 4, 64), (8, 1, 128), (2, 2, 64)), (0, 1)):
        fq = L.usp_attn_fwd_workspace_bytes(s_k, hq, hkv, d, BF16)
        bq = L.usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, BF16)
        f_min = vcopy(s_k, hkv, d)
        b_min = bq - dq_room(s_q, hq, hkv, d)
        for frac in (0.0, 0.3, 0.7, 1.0, 2.0):
            fw = int(f_min + frac * max(fq - f_min, s_q * hq * d * 8))
            z = L.usp_attn_fwd_num_splits(s_q, q_off, s_k, k_off, s_k, hq, hkv, d, causal, BF16, fw)
            assert z >= 1
            if z > 1:
                need = -(-z * s_q * hq * d * 4 // 256) * 256 + z * hq * s_q * 4
                assert f_min + need <= fw, (s_q, s_k, hq, hkv, d, causal, fw, z)
            bw = int(b_min + frac * max(bq - b_min, s_q * hq * d * 8))
            z = L.usp_attn_bwd_num_splits(s_q, q_off, s_k, k_off, s_k, hq, hkv, d, causal, BF16, bw)
            assert z >= 1
            if z > 1:
                assert b_min + z * s_q * hq * d * 4 <= bw, (s_q, s_k, hq, hkv, d, causal, bw, z)


def test_fast_division_host_side(tmp_path):
    """The pack/unpack kernels divide by run and row lengths with a
    multiply-high reciprocal; check it exhaustively on small values and on
    random 32-bit values, on the host."""
    src = tmp_path / "fastdiv.cpp"
    src.write_text(r'''
#include "usp_internal.h"
#include <cstdio>
#include <random>
int main() {
  std::mt19937_64 g(1);
  for (uint32_t d = 1; d < 5000; ++d) {
    usp::FastDiv f = usp::FastDiv::make(d);
    for (uint32_t n = 0; n < 20000; ++n) if (f.div(n) != n / d) { printf("bad %u %u\n", n, d); return 1; }
    for (int t = 0; t < 2000; ++t) { uint32_t n = (uint32_t)g(); if (f.div(n) != n / d) { printf("bad %u %u\n", n, d); return 1; } }
  }
  for (int t = 0; t < 200000; ++t) {
    uint32_t d = (uint32_t)(g() % 0x7fffffffu) + 1, n = (uint32_t)g();
    if (usp::FastDiv::make(d).div(n) != n / d) { printf("bad %u %u\n", n, d); return 1; }
  }
  printf("ok\n");
  return 0;
}
''')
    exe = tmp_path / "fastdiv"
    inc = os.path.join(ROOT, "ulysses_sequence_parallelism_amd", "csrc")
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", inc,
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


def bwd_na(L, s_pad=256, s_valid=256, cu=None, n_docs=0, hq=4, hkv=1, d=128, scale=0.088,
           causal=1, dt=BF16, ptrs=None):
    ptrs = ptrs or [A + (i << 26) for i in range(9)]
    return L.usp_attn_bwd_noalloc(*(ctypes.c_void_p(x) for x in ptrs), s_pad, s_valid,
                                  ctypes.c_void_p(cu), n_docs, hq, hkv, d, scale, causal, dt, None)


def test_noalloc_backward_rejects_on_the_host(L):
    """usp_attn_bwd_noalloc: the argument errors of usp_attn_bwd, and sizes
    whose required workspace exceeds the static array, all before any HIP call."""
    import ulysses_sequence_parallelism_amd as usp
    assert usp.USP_NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert re.search(r"#define USP_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)
    assert bwd_na(L, s_valid=0) == INVALID
    assert bwd_na(L, s_valid=257) == INVALID
    assert bwd_na(L, hq=6, hkv=4) == INVALID
    assert bwd_na(L, d=96) == UNSUPPORTED
    assert bwd_na(L, dt=7) == UNSUPPORTED
    assert bwd_na(L, scale=0.0) == INVALID
    p = [A + (i << 26) for i in range(9)]
    p[3] = 0
    assert bwd_na(L, ptrs=p) == NULLP
    p = [A + (i << 26) for i in range(9)]
    p[7] = p[1]  # dk aliases k
    assert bwd_na(L, ptrs=p) == INVALID
    p[7] = A + (7 << 26) + 8  # misaligned
    assert bwd_na(L, ptrs=p) == INVALID
    # required workspace beyond 32 MiB: 8192 rows on one KV head need 16 row
    # chunks of fp32 partial dK and dV (134 MB)
    need = L.usp_attn_bwd_workspace_bytes(8192, 4, 1, 128, BF16)
    assert need > (32 << 20)
    assert bwd_na(L, s_pad=8192, s_valid=8192) == WORKSPACE
    # D and LSE alone: 2^19 rows x 16 heads x 8 bytes = 64 MiB
    far = [A + (i << 32) for i in range(9)]
    assert bwd_na(L, s_pad=1 << 19, s_valid=1 << 19, hq=16, hkv=16, ptrs=far) == WORKSPACE
