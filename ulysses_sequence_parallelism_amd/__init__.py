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
    "usp_status_string",
    "usp_padded_len",
    "usp_pad_pack_seq2head",
    "usp_unpack_head2seq",
    "usp_attn_fwd_workspace_bytes",
    "usp_attn_fwd",
    "usp_attn_bwd_workspace_bytes",
    "usp_attn_bwd",
    "usp_trace_enable",
    "usp_trace_collect",
    "USP_BF16",
    "USP_FP32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libusp.so")
USP_BF16, USP_FP32 = 0, 1
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
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise UspError(fn, status)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise UspError("dtype", -2)
    return _DTYPES[t.dtype]


def usp_version() -> int:
    return lib().usp_version()


def usp_status_string(status: int) -> str:
    return lib().usp_status_string(status).decode()


def usp_padded_len(s_real: int, p: int) -> int:
    return lib().usp_padded_len(s_real, p)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


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
    _check("usp_pad_pack_seq2head",
           lib().usp_pad_pack_seq2head(_ptr(x), _ptr(out), s_real, p, h, d, _dtype(x),
                                       _stream(stream)))
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
    _check("usp_unpack_head2seq",
           lib().usp_unpack_head2seq(_ptr(y), _ptr(out), s_real, p, p * hp, d, _dtype(y),
                                     _stream(stream)))
    return out


def usp_attn_fwd_workspace_bytes(s_pad: int, hq: int, hkv: int, d: int, dtype: int) -> int:
    return lib().usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, dtype)


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
    o [s_pad, hq, d] in q's dtype and lse [hq, s_pad] fp32."""
    _contig(q, k, v)
    s_pad, hq, d = q.shape
    hkv = k.shape[1]
    s_valid = s_pad if s_valid is None else s_valid
    scale = float(d) ** -0.5 if softmax_scale is None else softmax_scale
    dt = _dtype(q)
    cu, n_docs = _cu(cu_seqlens, s_pad, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, s_pad), dtype=torch.float32, device=q.device)
    ws = _workspace(usp_attn_fwd_workspace_bytes(s_pad, hq, hkv, d, dt), q.device, workspace)
    _check("usp_attn_fwd", lib().usp_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), s_pad, s_valid, _ptr(cu), n_docs,
        hq, hkv, d, scale, int(causal), dt, _stream(stream)))
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
    cu, n_docs = _cu(cu_seqlens, s_pad, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws = _workspace(usp_attn_bwd_workspace_bytes(s_pad, hq, hkv, d, dt), q.device, workspace)
    _check("usp_attn_bwd", lib().usp_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s_pad, s_valid, _ptr(cu),
        n_docs, hq, hkv, d, scale, int(causal), dt, _stream(stream)))
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
