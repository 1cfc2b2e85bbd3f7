"""CPU-side checks of the Python binding: every tensor it hands to the C ABI
must have the shape and dtype the call assumes and be a GPU tensor (the
library sees only device pointers), and packed-document offsets are validated
on the host. All of these raise before any device call, so they run without a
GPU."""
import os

import pytest
import torch

import ulysses_sequence_parallelism_amd as usp


@pytest.fixture(autouse=True)
def _lib():
    if not os.path.exists(usp.LIB_PATH):
        pytest.skip("libusp.so not built")


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_forward_rejects_mismatched_outputs_and_inputs():
    q, k, v = bf(64, 4, 128), bf(64, 1, 128), bf(64, 1, 128)
    with pytest.raises(ValueError, match="out"):
        usp.usp_attn_fwd(q, k, v, out=bf(32, 4, 128))
    with pytest.raises(ValueError, match="lse"):
        usp.usp_attn_fwd(q, k, v, lse=f32(4, 63))
    with pytest.raises(ValueError, match="out"):
        usp.usp_attn_fwd(q, k, v, out=f32(64, 4, 128))          # fp32 O for bf16 inputs
    with pytest.raises(ValueError, match="k"):
        usp.usp_attn_fwd(q, bf(63, 1, 128), v)                  # K rows != Q rows
    with pytest.raises(ValueError, match="v"):
        usp.usp_attn_fwd(q, k, v.float())
    with pytest.raises(ValueError, match="contiguous"):
        usp.usp_attn_fwd(bf(4, 64, 128).transpose(0, 1), k, v)


def test_backward_rejects_mismatched_gradients():
    q, k, v = bf(64, 4, 128), bf(64, 1, 128), bf(64, 1, 128)
    o, do, lse = bf(64, 4, 128), bf(64, 4, 128), f32(4, 64)
    with pytest.raises(ValueError, match="dk"):
        usp.usp_attn_bwd(q, k, v, o, lse, do, dk=bf(64, 2, 128))
    with pytest.raises(ValueError, match="dq"):
        usp.usp_attn_bwd(q, k, v, o, lse, do, dq=f32(64, 4, 128))
    with pytest.raises(ValueError, match="lse"):
        usp.usp_attn_bwd(q, k, v, o, lse.to(torch.bfloat16), do)
    with pytest.raises(ValueError, match="dout"):
        usp.usp_attn_bwd(q, k, v, o, lse, bf(64, 2, 128))


def test_interval_calls_reject_mismatched_tensors():
    q, k, v = bf(40, 4, 128), bf(100, 1, 128), bf(100, 1, 128)
    with pytest.raises(ValueError, match="out"):
        usp.usp_attn_fwd_interval(q, k, v, q_off=10, out=f32(41, 4, 128))
    with pytest.raises(ValueError, match="lse"):
        usp.usp_attn_fwd_interval(q, k, v, lse=f32(4, 100))     # LSE is per query row
    with pytest.raises(ValueError, match="v"):
        usp.usp_attn_fwd_interval(q, k, bf(99, 1, 128))
    o, do, lse = bf(40, 4, 128), bf(40, 4, 128), f32(4, 40)
    with pytest.raises(ValueError, match="dk"):
        usp.usp_attn_bwd_interval(q, k, v, o, lse, do, dk=f32(40, 1, 128))  # dK is per key
    with pytest.raises(ValueError, match="dq"):
        usp.usp_attn_bwd_interval(q, k, v, o, lse, do, dq=f32(100, 4, 128))
    with pytest.raises(usp.UspError):  # bf16 and fp32 gradients mixed
        usp.usp_attn_bwd_interval(q, k, v, o, lse, do, dq=f32(40, 4, 128), dk=bf(100, 1, 128),
                                  dv=f32(100, 1, 128))


def test_merge_rejects_non_fp32_partials_and_bad_shapes():
    o, lse = f32(30, 4, 128), f32(4, 30)
    with pytest.raises(ValueError, match="o_a"):
        usp.usp_attn_merge(o.to(torch.bfloat16), lse, o, lse)
    with pytest.raises(ValueError, match="lse_b"):
        usp.usp_attn_merge(o, lse, o, f32(4, 31))
    with pytest.raises(ValueError, match="out"):
        usp.usp_attn_merge(o, lse, o, lse, out=f32(30, 4, 64))


def test_pack_unpack_reject_bad_outputs():
    x = bf(10, 8, 64)
    with pytest.raises(ValueError, match="out"):
        usp.usp_pad_pack_seq2head(x, 4, out=bf(4, 11, 2, 64))   # s_pad is 12
    with pytest.raises(ValueError, match="out"):
        usp.usp_pad_pack_seq2head(x, 4, out=f32(4, 12, 2, 64))
    with pytest.raises(ValueError, match="out"):
        usp.usp_unpack_head2seq(bf(4, 12, 2, 64), 10, out=bf(12, 8, 64))


@pytest.mark.parametrize("cu", [[1, 64], [0, 30, 20, 64], [0, 30, 63], [64], [[0, 64]]])
def test_document_offsets_validated_on_the_host(cu):
    q, k, v = bf(64, 4, 128), bf(64, 1, 128), bf(64, 1, 128)
    with pytest.raises(usp.UspError):
        usp.usp_attn_fwd(q, k, v, cu_seqlens=cu)


def test_interval_document_offsets_must_cover_the_call():
    q, k, v = bf(40, 4, 128), bf(100, 1, 128), bf(100, 1, 128)
    # global extent is max(q_off + 40, k_off + 100) = 150
    with pytest.raises(usp.UspError):
        usp.usp_attn_fwd_interval(q, k, v, q_off=110, k_off=50, cu_seqlens=[0, 70, 149])
    with pytest.raises(usp.UspError):
        usp.usp_attn_fwd_interval(q, k, v, q_off=0, k_off=0, cu_seqlens=[0, 50, 40, 150])


def test_host_tensors_are_refused_before_the_call():
    """Correct shapes and dtypes, but host tensors: a host pointer must never
    reach a kernel."""
    q, k, v = bf(64, 4, 128), bf(64, 1, 128), bf(64, 1, 128)
    o, do, lse = bf(64, 4, 128), bf(64, 4, 128), f32(4, 64)
    gpu = "must be on a GPU"
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_fwd(q, k, v)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_bwd(q, k, v, o, lse, do)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_bwd_noalloc(q, k, v, o, lse, do)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_fwd_interval(q, k, v)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_bwd_interval(q, k, v, o, lse, do)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_attn_merge(f32(64, 4, 128), lse, f32(64, 4, 128), lse)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_pad_pack_seq2head(bf(10, 8, 64), 4)
    with pytest.raises(ValueError, match=gpu):
        usp.usp_unpack_head2seq(bf(4, 12, 2, 64), 10)
