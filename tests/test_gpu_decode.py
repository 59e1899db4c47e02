"""GPU parity of fa_decode (split-key decode against a K/V cache) with the fp64 oracle.

The oracle is `oracle.attention.decode`: the rows are the last Nq positions of
the sequence of Nk keys; under the causal mask row i sees keys 0 .. Nk - Nq + i.
Bars as for the forward (bf16 O: max 2e-2, mean 2e-3; LSE relative 1e-5).
"""
import numpy as np
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.attention as ora
import synth
from gpu_helpers import check, check_lse, require_gpu, say, to_dev, to64

pytestmark = pytest.mark.gpu


def _inputs(B, Nq, Nk, H, d, seed, qk_mult=1.0):
    host = synth.make_decode_inputs(B, Nq, Nk, H, d, seed, qk_mult)
    dev = {x: to_dev(host[x]) for x in "qkv"}
    f64 = {x: synth.decode(host[x]) for x in "qkv"}
    return dev, f64


def _check_heads(o, lse, f64, scale, causal, heads, what):
    o64, lse64 = to64(o), to64(lse)
    for b, h in heads:
        o_ref, lse_ref = ora.decode(f64["q"][b, :, h], f64["k"][b, :, h], f64["v"][b, :, h], scale, causal)
        check(o64[b, :, h], o_ref, "bf16", f"{what} O (b={b}, h={h})")
        check_lse(lse64[b, h], lse_ref, f"{what} LSE (b={b}, h={h})")


CASES = [
    # B, Nq, Nk, H, d, causal, splits
    (1, 1, 1, 1, 64, True, 0),
    (1, 1, 31, 2, 64, False, 0),
    (2, 3, 33, 2, 64, True, 0),
    (1, 16, 500, 3, 128, True, 0),
    (2, 32, 4097, 2, 64, True, 0),
    (1, 5, 4097, 2, 128, False, 7),
    (1, 2, 300, 1, 64, True, 200),        # more chunks than 32-key blocks: empty chunks
    (1, 32, 32, 2, 128, True, 0),         # Nq = Nk: the square causal forward
    (2, 1, 70000, 2, 128, False, 0),
    (1, 4, 9000, 2, 64, True, 1),         # one chunk
]


@pytest.mark.parametrize("B,Nq,Nk,H,d,causal,splits", CASES)
def test_decode_matches_oracle(B, Nq, Nk, H, d, causal, splits):
    require_gpu()
    say("decode", B, Nq, Nk, H, d, causal, splits)
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=1000 + Nk + Nq)
    scale = synth.f32(d ** -0.5)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal, splits=splits)
    torch.cuda.synchronize()
    _check_heads(o, lse, f64, scale, causal, [(b, h) for b in range(B) for h in range(H)], "decode")


def test_decode_long_cache_all_heads():
    """A long cache: [B, Nk, H, d] = [4, 32768, 8, 128], one query row, all 32 heads."""
    require_gpu()
    B, Nq, Nk, H, d = 4, 1, 32768, 8, 128
    say("decode long cache", B, Nq, Nk, H, d)
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=7)
    scale = synth.f32(d ** -0.5)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    _check_heads(o, lse, f64, scale, True, [(b, h) for b in range(B) for h in range(H)], "long cache")


@pytest.mark.parametrize("Nq", [1, 4])
def test_decode_bench_shape_sampled_heads(Nq):
    """The bench's decode workload, [B, Nq, Nk, H, d] = [8, Nq, 32768, 32,
    128] causal, in the launch configuration it times (the library's chunk
    count: 4 chunks per head, 1024 workgroups); eight heads spread over the
    batch against the oracle."""
    require_gpu()
    B, Nk, H, d = 8, 32768, 32, 128
    say("decode bench shape", B, Nq, Nk, H, d)
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=11)
    scale = synth.f32(d ** -0.5)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    heads = [(b, (5 * b + 3) % H) for b in range(B)]
    _check_heads(o, lse, f64, scale, True, heads, "bench shape")


def test_decode_sharp_softmax():
    """Q and K doubled (logit standard deviation about 4): a few keys dominate."""
    require_gpu()
    B, Nq, Nk, H, d = 1, 8, 6000, 2, 128
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=8, qk_mult=2.0)
    scale = synth.f32(d ** -0.5)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    _check_heads(o, lse, f64, scale, True, [(0, 0), (0, 1)], "sharp")


def test_decode_split_counts_agree():
    """Any number of chunks gives the same result up to rounding."""
    require_gpu()
    B, Nq, Nk, H, d = 1, 4, 5000, 2, 64
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=9)
    scale = synth.f32(d ** -0.5)
    outs = []
    for splits in (1, 3, 16, 157):
        o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=True, splits=splits)
        torch.cuda.synchronize()
        _check_heads(o, lse, f64, scale, True, [(0, 0), (0, 1)], f"splits={splits}")
        outs.append((to64(o), to64(lse)))
    for o, lse in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 2e-2
        assert (np.abs(lse - outs[0][1]) / np.maximum(1.0, np.abs(outs[0][1]))).max() <= 2e-5


def test_decode_square_equals_forward():
    """Nq = Nk with the causal mask is the square causal forward."""
    require_gpu()
    B, N, H, d = 2, 32, 4, 64
    dev, _ = _inputs(B, N, N, H, d, seed=10)
    scale = synth.f32(d ** -0.5)
    o_d, lse_d = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    o_f, lse_f = fa.forward(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    assert np.abs(to64(o_d) - to64(o_f)).max() <= 2e-2
    assert (np.abs(to64(lse_d) - to64(lse_f)) / np.maximum(1.0, np.abs(to64(lse_f)))).max() <= 2e-5


def test_decode_zero_scale_is_uniform():
    """scale = 0: every visible key has the same weight."""
    require_gpu()
    B, Nq, Nk, H, d = 1, 3, 700, 1, 128
    dev, f64 = _inputs(B, Nq, Nk, H, d, seed=11)
    o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=0.0, causal=True)
    torch.cuda.synchronize()
    v = f64["v"][0, :, 0]
    for i in range(Nq):
        n_vis = Nk - Nq + i + 1
        check(to64(o)[0, i, 0], v[:n_vis].mean(axis=0), "bf16", f"uniform row {i}")
        check_lse(to64(lse)[0, 0, i], np.log(n_vis), f"uniform row {i} LSE")
