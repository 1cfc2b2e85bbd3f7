"""Shared helpers for the GPU parity tests (oracle on the CPU, kernels through
the C ABI)."""
import sys

import numpy as np
import torch

BF16_MAX, BF16_MEAN = 2e-2, 2e-3   # bf16 bar: max |err| and mean |err| per output tensor
FP32_MAX = 1e-4                    # fp32 bar: max |err|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    """torch tensor (any device, bf16/fp32) -> numpy float64 (exact up-cast)."""
    return t.detach().to("cpu", torch.float64).numpy()


BF16_HALF_ULP = 2.0 ** -9           # half a bf16 ulp, relative


def check_close(name, got, ref, dtype, bf16_out=None):
    """Compare GPU output (numpy f64) with the oracle (numpy f64) at the bar
    for the dtype; returns (max_abs, mean_abs).

    bf16 bar: max |err| <= 2e-2 and mean |err| <= 2e-3 per output tensor. When
    the output itself is stored in bf16 (O, dQ, dK, dV; not the fp32 LSE), both
    bars also allow the output format's own rounding, half a bf16 ulp of |ref|
    (2^-9 |ref|): element-wise for the max bar, its mean over the tensor for the
    mean bar. No bf16-output implementation can do better: an element of
    magnitude 8 has bf16 neighbours 0.0625 apart, and a tensor whose elements
    are mostly of magnitude 2-6 (dV of a one-token sequence, the sum of the
    heads' dO rows) has a mean rounding error above 2e-3 even when every
    element is the correctly rounded exact value."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU values"
    if bf16_out is None:
        bf16_out = dtype == "bf16" and not name.upper().startswith("LSE")
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    allow = BF16_MAX + (BF16_HALF_ULP * np.abs(ref) if bf16_out else 0.0)
    excess = float((err - allow).max()) if err.size else -1.0
    say(f"  {name}: max|err| {mx:.3e}  mean|err| {mean:.3e}  (max|ref| {np.abs(ref).max():.3e})")
    if dtype == "fp32":
        assert mx <= FP32_MAX, f"{name}: max|err| {mx} > {FP32_MAX}"
    else:
        assert excess <= 0.0, f"{name}: max|err| {mx} exceeds 2e-2 (+ bf16 half-ulp) by {excess}"
        mean_allow = BF16_MEAN + (float(np.mean(BF16_HALF_ULP * np.abs(ref))) if bf16_out and err.size else 0.0)
        assert mean <= mean_allow, f"{name}: mean|err| {mean} > {mean_allow} (2e-3 + mean bf16 half-ulp)"
    return mx, mean


def gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")
