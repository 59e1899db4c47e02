"""GPU parity of fa_forward_dropout / fa_backward_dropout with the dropout oracle.

The oracle replays the mask from (head, query row, key, seed, offset) with its
own Philox4x32-10 (oracle/dropout.py), so the comparison is element by element
against the same mask.  Bars: `gpu_helpers.check_dropout` with s =
keep_scale(p) (about 1 / (1 - p)), the multiplier of every kept term: 2^-8
|ref| plus s times the plain path's bars, plus for dQ and dK the bound of
`gpu_helpers.dropout_d_terms` on what the bf16 rounding of the stored O moves
them by through D = rowsum(dO * O).  A wrong mask element moves a short
row's result by a whole term, far above these bars; the bit-exact mask test
covers long rows.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.dropout as drop
import synth
from gpu_helpers import check_dropout, check_lse, dropout_d_terms, inputs, require_gpu, say, to64

pytestmark = pytest.mark.gpu

SEED = 0x5EED_0000_1234_ABCD


def check(got, ref, p, what, d_term=None):
    check_dropout(got, ref, drop.keep_scale(p), what, d_term)


def _run(shape, seed, causal, p, offset=0, heads=None, check_rows=None):
    require_gpu()
    B, N, H, d = shape
    say("dropout", shape, "causal", causal, "p", p, "offset", offset)
    dev, f64 = inputs(shape, "bf16", seed, with_do=True)
    scale = synth.f32(d ** -0.5)
    o, lse = fa.forward_dropout(dev["q"], dev["k"], dev["v"], p, SEED, offset, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_dropout(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, p, SEED, offset,
                                     scale=scale, causal=causal)
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        q, k, v, do = (f64[n][b, :, h] for n in ("q", "k", "v", "do"))
        keep = drop.keep_mask(b * H + h, np.arange(N), N, p, SEED, offset)
        o_r, lse_r = drop.forward(q, k, v, scale, causal, keep, p)
        check(to64(o[b, :, h]), o_r, p, f"dropout O b={b} h={h}")
        check_lse(to64(lse[b, h]), lse_r, f"dropout LSE b={b} h={h}")
        dq_r, dk_r, dv_r, _ = drop.backward(q, k, v, do, scale, causal, keep, p)
        dq_t, dk_t = dropout_d_terms(q, k, do, o_r, scale, causal)
        for name, got, ref, t in (("dQ", dq, dq_r, dq_t), ("dK", dk, dk_r, dk_t), ("dV", dv, dv_r, None)):
            check(to64(got[b, :, h]), ref, p, f"dropout {name} b={b} h={h}", t)
    return dev, (o, lse), (dq, dk, dv)


@pytest.mark.parametrize("d,N", [(64, 17), (64, 129), (64, 300), (128, 100), (128, 300), (256, 129)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_matches_oracle(d, N, causal, p):
    _run((2, N, 2, d), 7000 + N + d, causal, p)


def test_dropout_offset_and_head_groups():
    """B*H a multiple of 8 with a ragged tile, and a non-zero counter offset."""
    _run((2, 300, 4, 64), 7100, True, 0.2, offset=77)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_dropout_smallest_rate(d):
    """p = 2^-16 (threshold t = 1, the smallest rate that runs the dropout
    kernels: almost every element kept, multiplier 65536/65535) against the
    oracle; p = 0 runs the plain kernels instead (next test)."""
    _run((2, 300, 2, d), 7250 + d, True, 2.0 ** -16)


def test_dropout_p0_is_plain_attention():
    """A rate that rounds to t = 0 runs what fa_forward / fa_backward run."""
    require_gpu()
    dev, f64 = inputs((1, 200, 2, 64), "bf16", 7200, with_do=True)
    o, lse = fa.forward_dropout(dev["q"], dev["k"], dev["v"], 0.0, SEED, scale=0.125, causal=True)
    o0, lse0 = fa.forward(dev["q"], dev["k"], dev["v"], scale=0.125, causal=True)
    dq, dk, dv = fa.backward_dropout(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, 0.0, SEED,
                                     scale=0.125, causal=True)
    g0 = fa.backward(dev["q"], dev["k"], dev["v"], o0, dev["do"], lse0, scale=0.125, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, lse0), "p = 0 forward differs from fa_forward"
    for a, b in zip((dq, dk, dv), g0):
        assert torch.equal(a, b), "p = 0 backward differs from fa_backward"


def test_dropout_deterministic_and_seed_dependent():
    require_gpu()
    dev, _ = inputs((1, 256, 2, 64), "bf16", 7300)
    runs = [fa.forward_dropout(dev["q"], dev["k"], dev["v"], 0.3, s, off, scale=0.125, causal=False)[0]
            for s, off in ((SEED, 0), (SEED, 0), (SEED + 1, 0), (SEED, 1))]
    torch.cuda.synchronize()
    assert torch.equal(runs[0], runs[1]), "same seed and offset: different outputs"
    for other in runs[2:]:
        assert not torch.equal(runs[0], other), "a different seed or offset gave the same output"


def test_dropout_full_size_sampled_rows():
    """[2, 8192, 16, 64] causal, p = 0.1 (the fwd+bwd workload's shape): sampled
    rows of two heads of O and LSE against the oracle (causal row i = attention
    over keys 0..i, with the mask of row i)."""
    require_gpu()
    B, N, H, d = 2, 8192, 16, 64
    p, scale = 0.1, 0.125
    say("dropout full size", B, N, H, d)
    dev, f64 = inputs((B, N, H, d), "bf16", 5, with_do=True)
    o, lse = fa.forward_dropout(dev["q"], dev["k"], dev["v"], p, SEED, scale=scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, 16)]))
    for b, h in [(0, 0), (B - 1, H - 1)]:
        for i in rows:
            q = f64["q"][b, i:i + 1, h]
            k, v = f64["k"][b, :i + 1, h], f64["v"][b, :i + 1, h]
            keep = drop.keep_mask(b * H + h, [i], i + 1, p, SEED)
            o_r, lse_r = drop.forward(q, k, v, scale, False, keep, p)
            check(to64(o[b, i:i + 1, h]), o_r, p, f"dropout O b={b} h={h} row={i}")
            check_lse(to64(lse[b, h, i:i + 1]), lse_r, f"dropout LSE b={b} h={h} row={i}")
