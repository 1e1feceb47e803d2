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
