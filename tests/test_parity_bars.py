"""The parity check's bf16 rounding allowance (helpers.bf16_half_ulp) against
what rounding to bf16 actually does: torch's float32 -> bfloat16 conversion
(round to nearest even, the rounding of the kernels' fp32 results) never moves
a value by more than the allowance, and moves values halfway between two bf16
numbers by exactly it."""
import numpy as np
import torch

from helpers import bf16_half_ulp


def test_half_ulp_bounds_bf16_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.03, 1.0, 3.0, 50.0)])
    x = x.astype(np.float32).astype(np.float64)
    r = torch.from_numpy(x).float().to(torch.bfloat16).to(torch.float64).numpy()
    assert (np.abs(r - x) <= bf16_half_ulp(x)).all()
    # the largest observed error per binade reaches the bound (to 0.1%)
    for e in (-4, 0, 1, 2, 5):
        sel = (np.abs(x) >= 2.0 ** e) & (np.abs(x) < 2.0 ** (e + 1))
        ratio = (np.abs(r - x)[sel] / bf16_half_ulp(x[sel])).max()
        assert ratio > 0.999, (e, ratio)


def test_half_ulp_at_midpoints_and_values():
    # 4 + 2^-6 lies halfway between the bf16 neighbours 4 and 4 + 2^-5
    for lo, step in ((4.0, 2.0 ** -5), (2.0, 2.0 ** -6), (0.5, 2.0 ** -8), (1.0, 2.0 ** -7)):
        mid = lo + step / 2
        r = float(torch.tensor(mid, dtype=torch.float32).to(torch.bfloat16))
        assert abs(r - mid) == step / 2 == float(bf16_half_ulp(mid))
    assert float(bf16_half_ulp(2.0)) == 2.0 ** -7
    assert float(bf16_half_ulp(3.99)) == 2.0 ** -7
    assert float(bf16_half_ulp(4.0)) == 2.0 ** -6
    assert float(bf16_half_ulp(-0.2)) == 2.0 ** -11
