"""GPU parity of pad+pack / unpack against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import gpu, say

pytestmark = pytest.mark.gpu


def bits(t):
    """Raw bit pattern view (uint16 for bf16, int32 for fp32) as numpy."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


CASES = [
    # s_real, p, h, d, dtype
    (1, 8, 8, 128, torch.bfloat16),
    (7, 2, 4, 64, torch.float32),
    (100, 4, 8, 128, torch.bfloat16),
    (1023, 8, 32, 128, torch.bfloat16),
    (999, 3, 6, 64, torch.bfloat16),
    (513, 2, 8, 64, torch.float32),
    (77, 4, 4, 2, torch.float32),     # 8-byte runs
    (65, 2, 2, 1, torch.float32),     # 4-byte runs
    (300, 1, 4, 128, torch.bfloat16), # p = 1 is the identity
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_p{c[1]}_h{c[2]}_d{c[3]}" for c in CASES])
def test_pack_unpack_bit_exact(case):
    import ulysses_sequence_parallelism_amd as usp
    dev = gpu()
    s, p, h, d, dt = case
    x = torch.from_numpy(workloads.normal_f32(7, s, p, (s, h, d))).to(dt)
    y = usp.usp_pad_pack_seq2head(x.to(dev), p)
    torch.cuda.synchronize()
    ref = oracle.pad_pack_seq2head(bits(x), p)
    np.testing.assert_array_equal(bits(y), ref)
    back = usp.usp_unpack_head2seq(y, s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(back), bits(x))
    np.testing.assert_array_equal(bits(back), oracle.unpack_head2seq(ref, s))


def test_pack_overwrites_stale_padding():
    import ulysses_sequence_parallelism_amd as usp
    dev = gpu()
    s, p, h, d = 13, 4, 8, 128
    x = torch.randn(s, h, d, dtype=torch.bfloat16, device=dev)
    y = torch.full((p, 16, h // p, d), 7.0, dtype=torch.bfloat16, device=dev)
    usp.usp_pad_pack_seq2head(x, p, out=y)
    torch.cuda.synchronize()
    assert (y[:, s:] == 0).all()


@pytest.mark.parametrize("name", ["tiny", "s8k", "s32k", "s120k", "s120k_pad", "thd131k"])
def test_workload_pack_unpack(name):
    """Full-size Q, K, V of every workload: pack bit-exact against the oracle;
    unpack inverts it."""
    import ulysses_sequence_parallelism_amd as usp
    dev = gpu()
    w = workloads.WORKLOADS[name]
    for which, label in ((workloads.Q, "Q"), (workloads.K, "K"), (workloads.V, "V")):
        x = workloads.tensor(w, which)
        say(f"{name} {label} {tuple(x.shape)} -> pack p={w.p}")
        xd = x.to(dev)
        y = usp.usp_pad_pack_seq2head(xd, w.p)
        torch.cuda.synchronize()
        ref = oracle.pad_pack_seq2head(bits(x), w.p)
        assert y.shape == ref.shape
        assert np.array_equal(bits(y), ref)
        back = usp.usp_unpack_head2seq(y, w.s)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                           xd.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32))
        del xd, y, back
