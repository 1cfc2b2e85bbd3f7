"""GPU check of the optional buffer checks (usp_check_buffers): with them on,
a host pointer or a tensor range that leaves its device allocation is refused
before any launch. Every rejected call here also passes a zero-byte
workspace, which the forward refuses after the buffer checks: whichever check
refuses it, nothing is launched."""
import ctypes

import pytest
import torch

from tests.gpu_helpers import gpu, say

pytestmark = pytest.mark.gpu

OK, INVALID, WORKSPACE = 0, -1, -5


def _hip():
    """The HIP runtime already mapped into this process."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    pytest.skip("HIP runtime not mapped")


def test_buffer_checks_refuse_host_and_out_of_range_buffers():
    import ulysses_sequence_parallelism_amd as L
    dev = gpu()
    lib = L.lib()
    s, hq, hkv, d = 64, 4, 1, 128
    g = torch.Generator(device="cpu").manual_seed(3)
    q = torch.randn((s, hq, d), generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn((s, hkv, d), generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn((s, hkv, d), generator=g).to(torch.bfloat16).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((hq, s), dtype=torch.float32, device=dev)
    ws = torch.empty(L.usp_attn_fwd_workspace_bytes(s, hq, hkv, d, L.USP_BF16), dtype=torch.uint8,
                     device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def fwd(q_ptr, o_ptr, ws_bytes):
        return lib.usp_attn_fwd(
            ctypes.c_void_p(q_ptr), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(o_ptr), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
            ws_bytes, s, s, None, 0, hq, hkv, d, d ** -0.5, 1, L.USP_BF16, stream)

    hip = _hip()
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    buf = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(buf), 1 << 20) == 0
    prev = lib.usp_check_buffers(1)
    try:
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), buf) == 0
        o_bytes = o.numel() * o.element_size()
        # an output whose last half lies past the end of its allocation
        tail = (base.value + size.value - o_bytes // 2) & ~15
        host = torch.zeros((s, hq, d), dtype=torch.bfloat16)
        say(f"allocation {size.value} bytes; output {o_bytes} bytes at offset "
            f"{tail - base.value}")
        assert fwd(q.data_ptr(), o.data_ptr(), 0) == WORKSPACE   # buffers pass, workspace refused
        assert fwd(host.data_ptr(), o.data_ptr(), 0) == INVALID  # host memory
        assert fwd(q.data_ptr(), tail, 0) == INVALID             # range leaves the allocation
        lib.usp_check_buffers(0)
        assert fwd(q.data_ptr(), tail, 0) == WORKSPACE           # not checked when off
        lib.usp_check_buffers(1)
        # a valid call runs with the checks on, and gives the same result as with them off
        assert fwd(q.data_ptr(), o.data_ptr(), ws.numel()) == OK
        torch.cuda.synchronize()
        o_on = o.clone()
        lib.usp_check_buffers(0)
        assert fwd(q.data_ptr(), o.data_ptr(), ws.numel()) == OK
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_on.view(torch.int16))
    finally:
        lib.usp_check_buffers(prev)
        hip.hipFree(buf)
