"""The per-element bf16 bar of the GPU parity tests (tests/gpu_helpers.py),
pinned on the CPU: ulp_bf16 is the distance to the next bfloat16 value as
torch's bfloat16 type gives it, and the bar is 2e-2 below |x| = 4."""
import numpy as np
import torch

from gpu_helpers import BF16_MAX, bf16_bar, ulp_bf16


def _torch_spacing(x):
    """Distance from bf16(|x|) rounded down to a power-of-two binade start to
    the next bf16 value, from torch: the spacing at |x|."""
    a = torch.tensor(np.abs(x), dtype=torch.float64)
    lo = torch.exp2(torch.floor(torch.log2(a))).to(torch.bfloat16)   # exact power of two
    nxt = torch.nextafter(lo, torch.full_like(lo, float("inf")))
    return (nxt.double() - lo.double()).numpy()


def test_ulp_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(5000) * np.exp2(rng.integers(-30, 30, 5000))
    assert np.array_equal(ulp_bf16(x), _torch_spacing(x))
    assert ulp_bf16(1.0) == 2.0 ** -7 and ulp_bf16(5.26) == 2.0 ** -5 and ulp_bf16(-8.0) == 2.0 ** -4


def test_bar_is_absolute_below_four():
    x = np.linspace(-3.999, 3.999, 2001)
    assert (bf16_bar(x) == BF16_MAX).all()
    assert bf16_bar(4.0) == 2.0 ** -5 and bf16_bar(12.0) == 2.0 ** -4
