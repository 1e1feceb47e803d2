"""The parity bar's output-rounding allowance must be exactly what bf16
rounding can cost, no more: |x - bf16(x)| <= half_ulp(x), and values a bit
further away than half_ulp really are not representable."""
import numpy as np
import torch

from tests import parity


def test_half_ulp_bounds_bf16_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 5.0, 30.0)])
    r = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    hu = parity.half_ulp(x, torch.bfloat16)
    assert np.all(np.abs(x - r) <= hu * (1 + 1e-12))
    # the allowance is tight: some values round by more than 0.9 half-ulp
    assert np.mean(np.abs(x - r) > 0.9 * hu) > 0.05
    assert np.all(parity.half_ulp(x, torch.float32) == 0)
    assert parity.half_ulp(np.array([8.0]), torch.bfloat16)[0] == 2.0 ** -5


def test_rounding_allowance_only_where_bf16_cannot_meet_the_bar():
    """Below |ref| = 8 half a bf16 ulp is at most 2^-7 < 2e-2, so the raw
    2e-2 bar applies; from 8 on it is 2^-5 or more and is allowed on top."""
    ref = np.array([0.0, 0.3, 1.5, 3.9, 4.0, 7.99, 8.0, 12.0, 16.0, -9.0])
    a = parity.rounding_allowance(ref, torch.bfloat16)
    assert np.all(a[:6] == 0)
    assert np.all(a[6:] == parity.half_ulp(ref[6:], torch.bfloat16))
    assert a[6] == 2.0 ** -5 and a[8] == 2.0 ** -4
    assert np.all(parity.rounding_allowance(ref, torch.float32) == 0)


def test_asserted_output_error_is_raw_below_eight():
    """An error of 0.03 at |ref| = 5 fails the bar (it did not under a
    half-ulp allowance at every magnitude); the same error at |ref| = 10
    is within 2e-2 of the correctly rounded value and passes."""
    ref = np.array([5.0, 10.0])
    gpu = torch.tensor([5.03, 10.03], dtype=torch.float64)
    e = parity.out_errs(gpu.to(torch.bfloat16), ref)
    # bf16 rounds 5.03 to 5.03125 and 10.03 to 10.0 (spacing 2^-5 / 2^-4)
    assert abs(e["raw"] - 0.03125) < 1e-12
    assert e["asserted"] > parity.OUT_ATOL
    e10 = parity.out_errs(gpu[1:].to(torch.bfloat16), ref[1:])
    assert e10["asserted"] <= parity.OUT_ATOL
