"""Shared helpers for the GPU parity tests (oracle on the CPU, kernels through
the C ABI)."""
import sys

import numpy as np
import torch

BF16_MAX, BF16_MEAN = 2e-2, 2e-3   # bf16 bar: max |err| and mean |err| per output tensor
FP32_MAX = 1e-4                    # fp32 bar: max |err|
# Magnitude-relative bars (every dtype), next to the absolute ones: an output
# that is zero, rescaled or shifted fails them however small its values are
# (those mistakes give relative errors of 0.1 and more).
# The mean bar comes from the arithmetic of the bf16 path: the second matrix
# product of each output takes one operand rounded to bf16 (P for O and dV,
# dS = P (dP - D) for dQ and dK), 8 significant bits, so every term carries a
# relative rounding error of up to 2^-8 (about 1.7e-3 RMS over a binade), and
# dS also carries D_i = dO_i . O_i formed from the bf16-rounded O. Sums of
# such terms keep that relative error: measured mean|err| / mean|ref| is up to
# 1.7e-3 for O, 2.2e-3 for dQ and 2.6e-3 for dK. The bar is 5e-3, about twice
# that.
# The absolute floors are fp32 accumulation noise on outputs whose exact value
# is 0 (for example dK of a one-token sequence, where dS = P (dP - D) = 0).
REL_MAX, REL_MEAN = 2e-2, 5e-3
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


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits)


def check_close(name, got, ref, dtype, bf16_out=None, bound=None):
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
    bound (optional, same shape as ref): a per-element error bound derived
    from the arithmetic (see rounding_bound); an element's bar is the larger
    of the above and its bound.
    fp32: max |err| <= 1e-4.
    Every dtype also meets the magnitude-relative bars
    max |err| <= 2e-2 max |ref| + 1e-5 and mean |err| <= 5e-3 mean |ref| + 1e-6
    (derivation above)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU values"
    if bf16_out is None:  # LSE is fp32 on every path
        bf16_out = dtype == "bf16" and "LSE" not in name.upper()
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
        if bound is not None:
            bar = np.maximum(bar, np.asarray(bound, dtype=np.float64))
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


def rounding_bound(ref, abs_sum, n_roundings, bf16_output=True):
    """Per-element bound on the error of a bf16-output sum whose terms carry
    n_roundings bf16 operand roundings (relative error <= 2^-8 each), to
    first order: n_roundings * 2^-8 * abs_sum (abs_sum = the oracle's sum of
    the terms' absolute values, which bounds how far the roundings can move
    the sum), plus, for a bf16 output, one bf16 step (its own rounding and
    that of the rounded oracle value it is compared with).
    dV = sum_i P_ij dO_i: the kernel rounds P (1 rounding).
    dK = scale sum_i dS_ij q_i with dS = bf16(bf16(P) (dP - D)): 2 roundings
    of each term, and D = dO . O from the bf16 O, whose error (O's rounding
    and the forward's rounded P) the oracle's abs_sum carries as P_ij B_i."""
    ref = np.asarray(ref, dtype=np.float64)
    step = bf16_spacing(bf16_rne(ref)) if bf16_output else 0.0
    return step + n_roundings * U_BF16 * np.asarray(abs_sum, np.float64)
