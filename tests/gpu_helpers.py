"""Helpers shared by the GPU parity tests: device upload, decode and the bars.

Bars (per element, GPU value upcast to fp64 minus the oracle's fp64 value):
  fp32 tensors   max |err| <= 1e-5
  bf16 tensors   max |err| <= 2e-2 and mean |err| <= 2e-3
  LSE            |err| <= 1e-5 * max(1, |LSE|)   (relative, with an absolute
                 floor where LSE is near zero)
"""
import sys

import numpy as np
import pytest
import torch

import synth

F32_MAX = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
LSE_REL = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """Upload a synth tensor: bf16 bit patterns become a bf16 tensor, fp32 stays fp32."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got, ref, dtype, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_MAX, f"{what}: max abs err {err.max():.3e} > {F32_MAX}"
    else:
        assert err.max() <= BF16_MAX, f"{what}: max abs err {err.max():.3e} > {BF16_MAX}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3e} > {BF16_MEAN}"
    return float(err.max()), float(err.mean())


def check_lse(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert np.isfinite(got).all(), f"{what}: non-finite LSE"
    assert err.max() <= LSE_REL, f"{what}: LSE rel err {err.max():.3e} > {LSE_REL}"
    return float(err.max())


def inputs(shape, dtype, seed, with_do=False, qk_mult=1.0):
    host = synth.make_inputs(shape, dtype, seed, with_do=with_do, qk_mult=qk_mult)
    dev = {k: to_dev(v) for k, v in host.items()}
    f64 = {k: synth.decode(v) for k, v in host.items()}
    return dev, f64
