"""Ulysses sequence-parallel rank-share hot path on MI355X (gfx950).

A thin ctypes binding over libusp.so (include/usp.h). Functions named
``usp_*`` mirror the C entry points one to one; they take torch tensors that
already live on the GPU, marshal pointers, sizes and the current HIP stream,
and raise ``UspError`` on a non-zero status. Every step of the computation
runs in the library's HIP kernels; this module only allocates outputs and
workspaces with torch (device memory plumbing).

If libusp.so has not been built, every call raises ``RuntimeError``: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "UspError",
    "lib",
    "usp_version",
    "usp_check_buffers",
    "usp_status_string",
    "usp_padded_len",
    "usp_pad_pack_seq2head",
    "usp_unpack_head2seq",
    "usp_attn_fwd_workspace_bytes",
    "usp_attn_fwd",
    "usp_attn_bwd_workspace_bytes",
    "usp_attn_bwd",
    "usp_attn_bwd_noalloc",
    "USP_NOALLOC_SCRATCH_BYTES",
    "usp_attn_fwd_interval",
    "usp_attn_fwd_num_splits",
    "usp_attn_bwd_num_splits",
    "usp_attn_merge",
    "usp_attn_bwd_interval_workspace_bytes",
    "usp_attn_bwd_interval",
    "usp_trace_enable",
    "usp_trace_collect",
    "USP_BF16",
    "USP_FP32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libusp.so")
USP_BF16, USP_FP32 = 0, 1
USP_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/usp.h
_DTYPES = {torch.bfloat16: USP_BF16, torch.float32: USP_FP32}

_lib = None


class _TraceEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_longlong),
                ("total_ms", ctypes.c_double)]


class UspError(ValueError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {usp_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libusp.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libusp.so not built ({LIB_PATH}); run "
                "`python -m ulysses_sequence_parallelism_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_size_t)
        L.usp_version.restype = i32
        L.usp_version.argtypes = []
        L.usp_check_buffers.restype = i32
        L.usp_check_buffers.argtypes = [i32]
        L.usp_status_string.restype = ctypes.c_char_p
        L.usp_status_string.argtypes = [i32]
        L.usp_padded_len.restype = i64
        L.usp_padded_len.argtypes = [i64, i32]
        for name in ("usp_pad_pack_seq2head", "usp_unpack_head2seq"):
            fn = getattr(L, name)
            fn.restype = i32
            fn.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp]
        for name in ("usp_attn_fwd_workspace_bytes", "usp_attn_bwd_workspace_bytes"):
            fn = getattr(L, name)
            fn.restype = sz
            fn.argtypes = [i64, i32, i32, i32, i32]
        L.usp_attn_fwd.restype = i32
        L.usp_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i64, i64, vp, i32, i32, i32, i32,
                                   f32, i32, i32, vp]
        L.usp_trace_enable.restype = i32
        L.usp_trace_enable.argtypes = [i32]
        L.usp_trace_collect.restype = i32
        L.usp_trace_collect.argtypes = [ctypes.POINTER(_TraceEntry), i32]
        L.usp_attn_bwd.restype = i32
        L.usp_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, vp, i32,
                                   i32, i32, i32, f32, i32, i32, vp]
        L.usp_attn_bwd_noalloc.restype = i32
        L.usp_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, i32,
                                           i32, i32, i32, f32, i32, i32, vp]
        L.usp_attn_fwd_interval.restype = i32
        L.usp_attn_fwd_interval.argtypes = [vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i64, i64,
                                            vp, i32, i32, i32, i32, f32, i32, i32, i32, vp]
        L.usp_attn_fwd_num_splits.restype = i32
        L.usp_attn_fwd_num_splits.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32, i32, i32, sz]
        L.usp_attn_bwd_num_splits.restype = i32
        L.usp_attn_bwd_num_splits.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32, i32, i32, sz]
        L.usp_attn_merge.restype = i32
        L.usp_attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp]
        L.usp_attn_bwd_interval_workspace_bytes.restype = sz
        L.usp_attn_bwd_interval_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        L.usp_attn_bwd_interval.restype = i32
        L.usp_attn_bwd_interval.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64,
                                            i64, i64, i64, vp, i32, i32, i32, i32, f32, i32, i32,
                                            i32, i32, vp]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None, dev=None):
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif dev is not None and stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


def _on_gpu(fn, *ts):
    """The device of the call. Every tensor handed to the C ABI must be a GPU
    tensor, all on one device: the library takes raw device pointers, and a host
    pointer would reach a kernel."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{fn}: every tensor must be on a GPU (got one on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: tensors on {dev} and {t.device}; all must be on one GPU")
    return dev


def _call(fn, dev, stream, cfun, *args):
    """Call cfun(*args, stream) with dev as the current device."""
    with torch.cuda.device(dev):
        _check(fn, cfun(*args, _stream(stream, dev)))


def _check(fn: str, status: int):
    if status != 0:
        raise UspError(fn, status)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise UspError("dtype", -2)
    return _DTYPES[t.dtype]


def usp_version() -> int:
    return lib().usp_version()


def usp_check_buffers(on: bool | None = None) -> bool:
    """Turn the library's optional buffer checks on or off (None: leave them);
    returns the previous state (see usp.h)."""
    return bool(lib().usp_check_buffers(-1 if on is None else int(bool(on))))


def usp_status_string(status: int) -> str:
    return lib().usp_status_string(status).decode()


def usp_padded_len(s_real: int, p: int) -> int:
    return lib().usp_padded_len(s_real, p)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _shapes(fn, **named):
    """Every tensor must have exactly the shape the C call will assume (the
    library sees only pointers and sizes)."""
    for name, (t, shape) in named.items():
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _same_dtype(fn, dtype, **named):
    for name, t in named.items():
        if t.dtype != dtype:
            raise ValueError(f"{fn}: {name} is {t.dtype}, expected {dtype}")


def usp_pad_pack_seq2head(x: torch.Tensor, p: int, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """x [s_real, H, d] -> y [p, s_pad, H/p, d] (see usp.h)."""
    _contig(x)
    s_real, h, d = x.shape
    s_pad = usp_padded_len(s_real, p)
    if out is None:
        if p < 1 or h % p:
            raise UspError("usp_pad_pack_seq2head", -1)
        out = torch.empty((p, s_pad, h // p, d), dtype=x.dtype, device=x.device)
    _contig(out)
    if p >= 1 and h % p == 0:
        _shapes("usp_pad_pack_seq2head", out=(out, (p, s_pad, h // p, d)))
    _same_dtype("usp_pad_pack_seq2head", x.dtype, out=out)
    dev = _on_gpu("usp_pad_pack_seq2head", x, out)
    _call("usp_pad_pack_seq2head", dev, stream, lib().usp_pad_pack_seq2head,
          _ptr(x), _ptr(out), s_real, p, h, d, _dtype(x))
    return out


def usp_unpack_head2seq(y: torch.Tensor, s_real: int, out: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """y [p, s_pad, H/p, d] -> x [s_real, H, d] (see usp.h)."""
    _contig(y)
    p, s_pad, hp, d = y.shape
    if s_pad != usp_padded_len(s_real, p):
        raise UspError("usp_unpack_head2seq", -1)
    if out is None:
        out = torch.empty((s_real, p * hp, d), dtype=y.dtype, device=y.device)
    _contig(out)
    _shapes("usp_unpack_head2seq", out=(out, (s_real, p * hp, d)))
    _same_dtype("usp_unpack_head2seq", y.dtype, out=out)
    dev = _on_gpu("usp_unpack_head2seq", y, out)
    _call("usp_unpack_head2seq", dev, stream, lib().usp_unpack_head2seq,
          _ptr(y), _ptr(out), s_real, p, p * hp, d, _dtype(y))
    return out


def usp_attn_fwd_workspace_bytes(s_pad: int, hq: int, hkv: int, d: int, dtype: int) -> int:
    return lib().usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, dtype)


def usp_attn_fwd_num_splits(s_q: int, s_k: int, hq: int, hkv: int, d: int, dtype: int,
                            causal: bool = True, q_off: int = 0, k_off: int = 0,
                            s_k_valid: int | None = None, workspace_bytes: int | None = None) -> int:
    """Key splits the forward runs for these sizes (1: one pass). The default
    workspace is the one the binding allocates, usp_attn_fwd_workspace_bytes(s_k)."""
    if workspace_bytes is None:
        workspace_bytes = usp_attn_fwd_workspace_bytes(s_k, hq, hkv, d, dtype)
    n = lib().usp_attn_fwd_num_splits(s_q, q_off, s_k, k_off, s_k if s_k_valid is None else s_k_valid,
                                      hq, hkv, d, int(causal), dtype, workspace_bytes)
    if n < 1:
        raise UspError("usp_attn_fwd_num_splits", n)
    return n


def usp_attn_bwd_num_splits(s_q: int, s_k: int, hq: int, hkv: int, d: int, dtype: int,
                            causal: bool = True, q_off: int = 0, k_off: int = 0,
                            s_k_valid: int | None = None, workspace_bytes: int | None = None) -> int:
    """Key splits the dQ kernel runs for these sizes (1: one pass). The default
    workspace is the one the binding allocates for the backward."""
    if workspace_bytes is None:
        workspace_bytes = usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, dtype)
    n = lib().usp_attn_bwd_num_splits(s_q, q_off, s_k, k_off, s_k if s_k_valid is None else s_k_valid,
                                      hq, hkv, d, int(causal), dtype, workspace_bytes)
    if n < 1:
        raise UspError("usp_attn_bwd_num_splits", n)
    return n


def usp_attn_bwd_workspace_bytes(s_pad: int, hq: int, hkv: int, d: int, dtype: int) -> int:
    return lib().usp_attn_bwd_workspace_bytes(s_pad, hq, hkv, d, dtype)


def _cu(cu_seqlens, s_pad, device):
    """Validate packed-document offsets on the host, return (device int32
    tensor or None, n_docs)."""
    if cu_seqlens is None:
        return None, 0
    host = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
    if host.ndim != 1 or host.numel() < 2 or int(host[0]) != 0 or int(host[-1]) != s_pad \
            or bool((host[1:] < host[:-1]).any()):
        raise UspError("cu_seqlens", -1)
    return host.to(device=device, dtype=torch.int32), host.numel() - 1


def _cu_any(cu_seqlens, s_pad, device):
    """cu_seqlens as given: a device int32 tensor is passed as is (the caller
    has validated it; the kernels clamp every offset to the sequence, so a bad
    one cannot reach memory out of range). This is the form to use under graph
    capture, where host validation would copy. Anything else is validated on
    the host and copied to the device."""
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        if (cu_seqlens.dtype != torch.int32 or cu_seqlens.ndim != 1
                or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2):
            raise UspError("cu_seqlens", -1)
        return cu_seqlens, cu_seqlens.numel() - 1
    return _cu(cu_seqlens, s_pad, device)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def usp_attn_fwd(q, k, v, s_valid=None, cu_seqlens=None, causal=True, softmax_scale=None,
                 out=None, lse=None, workspace=None, stream=None):
    """Attention forward over one rank's share (see usp.h).

    q [s_pad, hq, d], k and v [s_pad, hkv, d]. Returns (o, lse) with
    o [s_pad, hq, d] in q's dtype and lse [hq, s_pad] fp32. cu_seqlens: a
    list or host tensor (validated here), or a device int32 tensor taken as
    is (the form for graph capture)."""
    _contig(q, k, v)
    s_pad, hq, d = q.shape
    hkv = k.shape[1]
    s_valid = s_pad if s_valid is None else s_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu_any(cu_seqlens, s_pad, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, s_pad), dtype=torch.float32, device=q.device)
    _contig(out, lse)
    _shapes("usp_attn_fwd", k=(k, (s_pad, hkv, d)), v=(v, (s_pad, hkv, d)), out=(out, q.shape),
            lse=(lse, (hq, s_pad)))
    _same_dtype("usp_attn_fwd", q.dtype, k=k, v=v, out=out)
    _same_dtype("usp_attn_fwd", torch.float32, lse=lse)
    ws = _workspace(usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, dt), q.device, workspace)
    dev = _on_gpu("usp_attn_fwd", q, k, v, out, lse, ws, cu)
    _call("usp_attn_fwd", dev, stream, lib().usp_attn_fwd,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), s_pad, s_valid, _ptr(cu), n_docs,
        hq, hkv, d, scale, int(causal), dt)
    return out, lse


def usp_attn_bwd(q, k, v, o, lse, dout, s_valid=None, cu_seqlens=None, causal=True,
                 softmax_scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward (see usp.h). Returns (dq, dk, dv)."""
    _contig(q, k, v, o, lse, dout)
    s_pad, hq, d = q.shape
    hkv = k.shape[1]
    s_valid = s_pad if s_valid is None else s_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu_any(cu_seqlens, s_pad, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _contig(dq, dk, dv)
    kshape = (s_pad, hkv, d)
    _shapes("usp_attn_bwd", k=(k, kshape), v=(v, kshape), o=(o, q.shape), dout=(dout, q.shape),
            lse=(lse, (hq, s_pad)), dq=(dq, q.shape), dk=(dk, kshape), dv=(dv, kshape))
    _same_dtype("usp_attn_bwd", q.dtype, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    _same_dtype("usp_attn_bwd", torch.float32, lse=lse)
    ws = _workspace(usp_attn_bwd_workspace_bytes(s_pad, hq, hkv, d, dt), q.device, workspace)
    dev = _on_gpu("usp_attn_bwd", q, k, v, o, lse, dout, dq, dk, dv, ws, cu)
    _call("usp_attn_bwd", dev, stream, lib().usp_attn_bwd,
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s_pad, s_valid, _ptr(cu),
        n_docs, hq, hkv, d, scale, int(causal), dt)
    return dq, dk, dv


def usp_attn_bwd_noalloc(q, k, v, o, lse, dout, s_valid=None, cu_seqlens=None, causal=True,
                         softmax_scale=None, dq=None, dk=None, dv=None, stream=None):
    """usp_attn_bwd with the library's own static workspace (see usp.h): the
    library allocates nothing. Pass dq, dk, dv to allocate nothing here either
    (cu_seqlens, if given, should then be a device int32 tensor). Returns
    (dq, dk, dv)."""
    _contig(q, k, v, o, lse, dout)
    s_pad, hq, d = q.shape
    hkv = k.shape[1]
    s_valid = s_pad if s_valid is None else s_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu_any(cu_seqlens, s_pad, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _contig(dq, dk, dv)
    kshape = (s_pad, hkv, d)
    _shapes("usp_attn_bwd_noalloc", k=(k, kshape), v=(v, kshape), o=(o, q.shape),
            dout=(dout, q.shape), lse=(lse, (hq, s_pad)), dq=(dq, q.shape), dk=(dk, kshape),
            dv=(dv, kshape))
    _same_dtype("usp_attn_bwd_noalloc", q.dtype, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    _same_dtype("usp_attn_bwd_noalloc", torch.float32, lse=lse)
    dev = _on_gpu("usp_attn_bwd_noalloc", q, k, v, o, lse, dout, dq, dk, dv, cu)
    _call("usp_attn_bwd_noalloc", dev, stream, lib().usp_attn_bwd_noalloc,
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        s_pad, s_valid, _ptr(cu), n_docs, hq, hkv, d, scale, int(causal), dt)
    return dq, dk, dv


def usp_trace_enable(on: bool = True) -> bool:
    """Turn kernel tracing on or off; returns the previous setting."""
    return bool(lib().usp_trace_enable(int(on)))


def usp_trace_collect(max_entries: int = 64) -> list[dict]:
    """Per-kernel launch counts and summed HIP-event durations recorded since
    the last collect, sorted by total time (waits for the recorded events)."""
    buf = (_TraceEntry * max_entries)()
    n = lib().usp_trace_collect(buf, max_entries)
    if n < 0:
        raise UspError("usp_trace_collect", n)
    return [{"name": buf[i].name.decode(), "launches": int(buf[i].launches),
             "total_ms": float(buf[i].total_ms)} for i in range(n)]


def _cu_global(cu_seqlens, extent, device):
    """Validate document offsets over global positions on the host: they start
    at 0, never decrease and cover every position the call touches."""
    if cu_seqlens is None:
        return None, 0
    host = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
    if host.ndim != 1 or host.numel() < 2 or int(host[0]) != 0 or int(host[-1]) < extent \
            or bool((host[1:] < host[:-1]).any()):
        raise UspError("cu_seqlens", -1)
    return host.to(device=device, dtype=torch.int32), host.numel() - 1


def usp_attn_fwd_interval(q, k, v, q_off=0, k_off=0, s_k_valid=None, cu_seqlens=None,
                          causal=True, softmax_scale=None, out_dtype=torch.float32, out=None,
                          lse=None, workspace=None, stream=None):
    """Attention of query rows at global positions q_off + [0, s_q) against keys
    at k_off + [0, s_k) (see usp.h). q [s_q, hq, d], k and v [s_k, hkv, d].
    Returns (o [s_q, hq, d] in out_dtype, lse [hq, s_q] fp32); rows without an
    allowed key get o = 0, lse = -inf."""
    _contig(q, k, v)
    s_q, hq, d = q.shape
    s_k, hkv = k.shape[0], k.shape[1]
    s_k_valid = s_k if s_k_valid is None else s_k_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu_global(cu_seqlens, max(q_off + s_q, k_off + s_k), q.device)
    if out is None:
        out = torch.empty((s_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, s_q), dtype=torch.float32, device=q.device)
    _contig(out, lse)
    _shapes("usp_attn_fwd_interval", v=(v, k.shape), out=(out, q.shape), lse=(lse, (hq, s_q)))
    _same_dtype("usp_attn_fwd_interval", q.dtype, k=k, v=v)
    _same_dtype("usp_attn_fwd_interval", torch.float32, lse=lse)
    ws = _workspace(usp_attn_fwd_workspace_bytes(s_k, hq, hkv, d, dt), q.device, workspace)
    dev = _on_gpu("usp_attn_fwd_interval", q, k, v, out, lse, ws, cu)
    _call("usp_attn_fwd_interval", dev, stream, lib().usp_attn_fwd_interval,
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), s_q, q_off, s_k, k_off, s_k_valid,
        _ptr(cu), n_docs, hq, hkv, d, scale, int(causal), dt, _dtype(out))
    return out, lse


def usp_attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse=None, out_dtype=torch.float32,
                   stream=None):
    """Exact log-sum-exp merge of two fp32 partials over disjoint key sets (see
    usp.h). out / lse may be o_a / lse_a themselves (in-place accumulation).
    Returns (o [s_q, hq, d] in out's dtype, lse [hq, s_q])."""
    _contig(o_a, lse_a, o_b, lse_b)
    s_q, hq, d = o_a.shape
    if out is None:
        out = torch.empty((s_q, hq, d), dtype=out_dtype, device=o_a.device)
    if lse is None:
        lse = torch.empty((hq, s_q), dtype=torch.float32, device=o_a.device)
    _contig(out, lse)
    _shapes("usp_attn_merge", o_b=(o_b, o_a.shape), lse_a=(lse_a, (hq, s_q)),
            lse_b=(lse_b, (hq, s_q)), out=(out, o_a.shape), lse=(lse, (hq, s_q)))
    _same_dtype("usp_attn_merge", torch.float32, o_a=o_a, o_b=o_b, lse_a=lse_a, lse_b=lse_b,
                lse=lse)
    dev = _on_gpu("usp_attn_merge", o_a, lse_a, o_b, lse_b, out, lse)
    _call("usp_attn_merge", dev, stream, lib().usp_attn_merge,
        _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out), _ptr(lse), s_q, hq, d,
        _dtype(out))
    return out, lse


def usp_attn_bwd_interval_workspace_bytes(s_q: int, s_k: int, hq: int, hkv: int, d: int,
                                          dtype: int) -> int:
    return lib().usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, dtype)


def usp_attn_bwd_interval(q, k, v, o, lse, dout, q_off=0, k_off=0, s_k_valid=None,
                          cu_seqlens=None, causal=True, softmax_scale=None,
                          grad_dtype=torch.float32, accumulate=False, dq=None, dk=None, dv=None,
                          workspace=None, stream=None):
    """Backward contributions of one (query interval, key interval) pair given
    the FINAL o and lse of the rows (see usp.h). With accumulate the fp32
    gradients are added to dq / dk / dv (allocated as zeros when not given).
    Returns (dq, dk, dv)."""
    _contig(q, k, v, o, lse, dout)
    s_q, hq, d = q.shape
    s_k, hkv = k.shape[0], k.shape[1]
    s_k_valid = s_k if s_k_valid is None else s_k_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu_global(cu_seqlens, max(q_off + s_q, k_off + s_k), q.device)
    alloc = torch.zeros if accumulate else torch.empty
    dq = alloc((s_q, hq, d), dtype=grad_dtype, device=q.device) if dq is None else dq
    dk = alloc((s_k, hkv, d), dtype=grad_dtype, device=q.device) if dk is None else dk
    dv = alloc((s_k, hkv, d), dtype=grad_dtype, device=q.device) if dv is None else dv
    _contig(dq, dk, dv)
    _shapes("usp_attn_bwd_interval", v=(v, k.shape), o=(o, q.shape), dout=(dout, q.shape),
            lse=(lse, (hq, s_q)), dq=(dq, q.shape), dk=(dk, k.shape), dv=(dv, k.shape))
    _same_dtype("usp_attn_bwd_interval", q.dtype, k=k, v=v, o=o, dout=dout)
    _same_dtype("usp_attn_bwd_interval", torch.float32, lse=lse)
    gdt = _dtype(dq)
    if _dtype(dk) != gdt or _dtype(dv) != gdt:
        raise UspError("usp_attn_bwd_interval", -1)
    ws = _workspace(usp_attn_bwd_interval_workspace_bytes(s_q, s_k, hq, hkv, d, dt), q.device,
                    workspace)
    dev = _on_gpu("usp_attn_bwd_interval", q, k, v, o, lse, dout, dq, dk, dv, ws, cu)
    _call("usp_attn_bwd_interval", dev, stream, lib().usp_attn_bwd_interval,
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s_q, q_off, s_k, k_off,
        s_k_valid, _ptr(cu), n_docs, hq, hkv, d, scale, int(causal), dt, gdt, int(accumulate))
    return dq, dk, dv
