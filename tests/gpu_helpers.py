"""Shared helpers for the GPU parity tests (oracle on the CPU, kernels through
the C ABI)."""
import sys

import numpy as np
import torch

BF16_MAX, BF16_MEAN = 2e-2, 2e-3   # bf16 bar: max |err| and mean |err| per output tensor
FP32_MAX = 1e-4                    # fp32 bar: max |err|
# Magnitude-relative bars (every dtype), next to the absolute ones: an output
# that is zero, rescaled or shifted fails them however small its values are.
# The absolute floors are fp32 accumulation noise on outputs whose exact value
# is 0 (for example dK of a one-token sequence, where dS = P (dP - D) = 0).
REL_MAX, REL_MEAN = 2e-2, 2e-3
REL_MAX_FLOOR, REL_MEAN_FLOOR = 1e-5, 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    """torch tensor (any device, bf16/fp32) -> numpy float64 (exact up-cast)."""
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_rne(x):
    """float64 values rounded to the nearest bfloat16 (ties to even) in ONE
    step, returned as float64. Going through float32 rounds twice; the two
    differ only where the float32 value lands exactly on a bfloat16 midpoint
    while the float64 value does not, and there the float64 value decides."""
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    low = b & 0xFFFF
    tie_in_f32 = (low == 0x8000) & (x32.astype(np.float64) != x)
    # ordinary round-to-nearest-even on the float32 bits
    even = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    # float32 tie that was not a float64 tie: away from zero iff |x| > |x32|
    up = (b + 0x8000) & 0xFFFF0000
    down = b & 0xFFFF0000
    away = np.abs(x) > np.abs(x32.astype(np.float64))
    r = np.where(tie_in_f32, np.where(away, up, down), even)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_spacing(x):
    """Distance from |x| (a bfloat16 value) to the next larger bfloat16."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, e - 8)


def check_close(name, got, ref, dtype, bf16_out=None):
    """Compare GPU output (numpy f64) with the exact oracle value (numpy f64)
    at the bar for the dtype; returns (max_abs, mean_abs) of the compared
    error.

    bf16 inputs: max |err| <= 2e-2 and mean |err| <= 2e-3 per output tensor.
    When the output itself is stored in bf16 (O, dQ, dK, dV; not the fp32 LSE
    or fp32 partials) it is compared with the oracle's value rounded to bf16
    (round to nearest even), the correctly rounded result. One exception: an
    element whose rounded value is 4 or more in magnitude, where neighbouring
    bf16 values are 2^-5 = 0.031 or more apart, may differ by one bf16 step,
    since an fp32 accumulation that is not itself exact can land on the other
    side of a rounding midpoint.
    fp32: max |err| <= 1e-4.
    Every dtype also meets the magnitude-relative bars
    max |err| <= 2e-2 max |ref| + 1e-5 and mean |err| <= 2e-3 mean |ref| + 1e-6."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU values"
    if bf16_out is None:
        bf16_out = dtype == "bf16" and not name.upper().startswith("LSE")
    if got.size == 0:
        return 0.0, 0.0
    ref_c = bf16_rne(ref) if (dtype == "bf16" and bf16_out) else ref
    err = np.abs(got - ref_c)
    mx, mean = float(err.max()), float(err.mean())
    amax, amean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    say(f"  {name}: max|err| {mx:.3e}  mean|err| {mean:.3e}  (max|ref| {amax:.3e}, "
        f"mean|ref| {amean:.3e}; rel max {mx / max(amax, 1e-300):.2e} "
        f"rel mean {mean / max(amean, 1e-300):.2e})")
    if dtype == "fp32":
        assert mx <= FP32_MAX, f"{name}: max|err| {mx} > {FP32_MAX}"
    else:
        bar = BF16_MAX
        if bf16_out:
            bar = np.maximum(BF16_MAX, np.where(np.abs(ref_c) >= 4.0, bf16_spacing(ref_c), 0.0))
        excess = float((err - bar).max())
        assert excess <= 0.0, f"{name}: max|err| {mx} exceeds the bar by {excess}"
        assert mean <= BF16_MEAN, f"{name}: mean|err| {mean} > {BF16_MEAN}"
    assert mx <= REL_MAX * amax + REL_MAX_FLOOR, \
        f"{name}: max|err| {mx} > {REL_MAX} max|ref| ({amax}) + {REL_MAX_FLOOR}"
    assert mean <= REL_MEAN * amean + REL_MEAN_FLOOR, \
        f"{name}: mean|err| {mean} > {REL_MEAN} mean|ref| ({amean}) + {REL_MEAN_FLOOR}"
    return mx, mean


def gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")
