"""CPU checks of the parity checker itself (tests/gpu_helpers.check_close):
the one-step bf16 rounding of the oracle values, and that a GPU result which
is zero, rescaled by 1.1 or shifted by one row fails the bars even when the
values are far below the absolute 2e-2 bar (as dK / dV are at 120K tokens)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import bf16_rne, bf16_spacing, check_close


def test_bf16_rne_matches_torch_on_float32_values():
    g = np.random.default_rng([5, 0, 1])
    x = np.concatenate([g.standard_normal(100000) * s for s in (1e-3, 1.0, 7.0, 300.0)])
    x = x.astype(np.float32)
    # every float32 bf16 tie pattern, both signs
    ties = (g.integers(0, 1 << 15, size=2000).astype(np.uint32) << 16) | 0x8000
    ties = np.concatenate([ties, ties | 0x80000000]).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_rne(x.astype(np.float64)), want)


def test_bf16_rne_rounds_float64_in_one_step():
    # 1 + 2^-8 is a bf16 midpoint (between 1 and 1 + 2^-7): a tie, to even (1.0)
    assert bf16_rne(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # just above the midpoint: float32 rounds it onto the midpoint, and a second
    # rounding would go to even (1.0); the single rounding goes up
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(x) == np.float32(1 + 2.0 ** -8)
    assert bf16_rne(np.array([x]))[0] == 1 + 2.0 ** -7
    assert bf16_rne(np.array([-x]))[0] == -(1 + 2.0 ** -7)
    # just below the next midpoint up (1 + 3 * 2^-8, which ties to even upwards)
    y = 1 + 3 * 2.0 ** -8 - 2.0 ** -40
    assert bf16_rne(np.array([y]))[0] == 1 + 2.0 ** -7
    assert bf16_spacing(np.array([1.0, 4.0, 7.9375, -8.0]))[1] == 2.0 ** -5
    assert bf16_spacing(np.array([1.0]))[0] == 2.0 ** -7


def _reference(s=300, hq=4, hkv=1, d=64, seed=(6, 0, 0)):
    g = np.random.default_rng(list(seed))
    q, k, v, do = (g.standard_normal((s, h, d)).astype(np.float32).astype(np.float64)
                   for h in (hq, hkv, hkv, hq))
    o, lse = oracle.attn_fwd(q, k, v, d ** -0.5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, lse, do, d ** -0.5)
    return {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}


@pytest.mark.parametrize("scale", [1.0, 1e-3])
def test_checker_accepts_rounded_and_rejects_planted_mistakes(scale):
    """A correctly rounded result passes; zeroed, 1.1x and row-shifted results
    fail, also when every value is 1e-3 of its size (far below 2e-2)."""
    ref = _reference()
    for name in ("O", "dQ", "dK", "dV"):
        r = ref[name] * scale
        check_close(name, bf16_rne(r), r, "bf16")          # the correctly rounded result
        check_close(name, r, r, "bf16", bf16_out=False)    # an fp32 output
        for bad in (np.zeros_like(r), 1.1 * r, np.roll(r, 1, axis=0)):
            with pytest.raises(AssertionError):
                check_close(name, bf16_rne(bad), r, "bf16")
    lse = ref["LSE"]
    check_close("LSE", lse, lse, "bf16")
    for bad in (np.zeros_like(lse), 1.1 * lse, np.roll(lse, 1, axis=1)):
        with pytest.raises(AssertionError):
            check_close("LSE", bad, lse, "bf16")


def test_checker_one_step_exception_only_at_four_and_up():
    # five probed elements among many small ones, so that the mean bar holds
    r = np.concatenate([[3.9, 4.1, 6.0, 9.0, 0.5], np.linspace(-0.3, 0.3, 200)])
    got = bf16_rne(r)
    check_close("v", got, r, "bf16")
    # one bf16 step away is allowed at |value| >= 4 only
    step = bf16_spacing(got)
    for i, ok in enumerate([False, True, True, True, False]):
        bad = got.copy()
        bad[i] += step[i] if ok else 2.5e-2
        if ok:
            check_close("v", bad, r, "bf16")
        else:
            with pytest.raises(AssertionError):
                check_close("v", bad, r, "bf16")
    # two steps are not
    bad = got.copy()
    bad[2] += 2 * step[2]
    with pytest.raises(AssertionError):
        check_close("v", bad, r, "bf16")


def test_checker_bound_widens_elements_not_the_tensor_bars():
    """A per-element rounding bound lets single large-magnitude elements
    differ by more than 2e-2, but a zeroed, rescaled or shifted tensor still
    fails the magnitude-relative bars."""
    from tests.gpu_helpers import rounding_bound
    ref = _reference()["dK"]
    abs_sum = 4.0 * np.abs(ref) + 0.5          # terms of mixed sign: larger than |ref|
    bound = rounding_bound(ref, abs_sum, 2)
    got = bf16_rne(ref)
    i = np.unravel_index(np.argmax(np.where(np.abs(ref) < 3.9, np.abs(ref), 0)), ref.shape)
    assert np.abs(ref[i]) > 1.0
    got[i] += 0.03 * np.sign(ref[i])            # one element off by 0.03, inside its bound
    assert bound[i] > 0.03
    with pytest.raises(AssertionError):
        check_close("dK", got, ref, "bf16")
    check_close("dK", got, ref, "bf16", bound=bound)
    for bad in (np.zeros_like(ref), 1.1 * ref, np.roll(ref, 1, axis=0)):
        with pytest.raises(AssertionError):
            check_close("dK", bf16_rne(bad), ref, "bf16", bound=bound)
