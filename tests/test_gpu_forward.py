"""GPU forward (fa_forward / fa_forward_f32) against the fp64 CPU oracle."""
import numpy as np
import pytest
import torch

import oracle.attention as ora
import synth
from gpu_helpers import check, check_lse, inputs, require_gpu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import exact_io_aware_39_amd as fa
    fa.load()


def fa_mod():
    import exact_io_aware_39_amd as fa
    return fa


def run_and_check(shape, dtype, seed, causal, scale, heads=None, rows_of=None, qk_mult=1.0, tag=""):
    fa = fa_mod()
    say(f"forward {tag} shape={shape} dtype={dtype} causal={causal} seed={seed} scale={scale}")
    dev, f64 = inputs(shape, dtype, seed, qk_mult=qk_mult)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    B, N, H, d = shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    worst = []
    for b, h in heads:
        q, k, v = f64["q"][b, :, h], f64["k"][b, :, h], f64["v"][b, :, h]
        if rows_of is None:
            o_ref, l_ref = ora.forward(q, k, v, scale, causal)
            o_got = to64(o[b, :, h])
            l_got = to64(lse[b, h])
        else:
            rows = rows_of(h)
            o_ref, l_ref = ora.forward_rows(q[rows], rows, k, v, scale, causal)
            o_got = to64(o[b, torch.as_tensor(rows, device=o.device), h])
            l_got = to64(lse[b, h, torch.as_tensor(rows, device=o.device)])
        worst.append(check(o_got, o_ref, dtype, f"O b={b} h={h} {tag}"))
        check_lse(l_got, l_ref, f"LSE b={b} h={h} {tag}")
    say(f"  ok: worst max/mean abs err O = {max(w[0] for w in worst):.3e} / {max(w[1] for w in worst):.3e}")
    return o, lse


def test_c1_fp32():
    w = synth.WORKLOADS["c1"]
    run_and_check(w.shape, w.dtype, w.seed, False, w.scale, tag="c1")


def test_c2_bf16_causal():
    w = synth.WORKLOADS["c2"]
    run_and_check(w.shape, w.dtype, w.seed, True, w.scale, tag="c2")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_small_ragged_bf16(N, d, causal):
    run_and_check((2, N, 3, d), "bf16", 1000 + N + d, causal, d ** -0.5, tag="ragged")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_head_groups_ragged(d, causal):
    """B*H a multiple of 8 (whole heads per XCD group) with a ragged last tile."""
    run_and_check((2, 300, 4, d), "bf16", 9009 + d, causal, d ** -0.5, tag="groups")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 33, 200, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_small_ragged_fp32(N, d, causal):
    run_and_check((2 if N > 300 else 1, N, 2, d), "f32", 2000 + N + d, causal, d ** -0.5, tag="ragged-f32")


@pytest.mark.parametrize("causal", [False, True])
def test_c3(causal):
    w = synth.WORKLOADS["c3"]
    run_and_check(w.shape, w.dtype, w.seed, causal, w.scale, heads=synth.checked_heads(w), tag="c3")


def test_c4_sampled_rows():
    w = synth.WORKLOADS["c4"]
    run_and_check(w.shape, w.dtype, w.seed, True, w.scale, rows_of=lambda h: synth.checked_rows(w, h),
                  qk_mult=w.qk_mult, tag="c4")


def test_c5_forward():
    w = synth.WORKLOADS["c5"]
    run_and_check(w.shape, w.dtype, w.seed, True, w.scale, heads=synth.checked_heads(w), tag="c5")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_invariants(d, causal):
    """V = 1 gives O = 1; (2Q, scale/2) is bit-identical to (Q, scale); reruns are bit-identical."""
    fa = fa_mod()
    shape = (2, 777, 4, d)
    say(f"invariants d={d} causal={causal} shape={shape}")
    dev, _ = inputs(shape, "bf16", 77 + d, qk_mult=1.0)
    q, k, v = dev["q"], dev["k"], dev["v"]
    ones = torch.ones_like(v)
    o1, _ = fa.forward(q, k, ones, scale=0.1, causal=causal)
    assert (o1.float() - 1).abs().max().item() <= 2 ** -7
    a_o, a_l = fa.forward(q, k, v, scale=0.1, causal=causal)
    b_o, b_l = fa.forward(q * 2, k, v, scale=0.05, causal=causal)
    c_o, c_l = fa.forward(q, k, v, scale=0.1, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
    assert torch.equal(a_o, c_o) and torch.equal(a_l, c_l)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform_attention(causal):
    fa = fa_mod()
    shape = (1, 150, 2, 64)
    say(f"zero scale causal={causal}")
    dev, f64 = inputs(shape, "bf16", 5150)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=0.0, causal=causal)
    v = f64["v"]
    for h in range(2):
        if causal:
            ref = np.cumsum(v[0, :, h], axis=0) / np.arange(1, 151)[:, None]
            lref = np.log(np.arange(1, 151))
        else:
            ref = np.tile(v[0, :, h].mean(axis=0), (150, 1))
            lref = np.full(150, np.log(150))
        check(to64(o[0, :, h]), ref, "bf16", f"zero-scale O h={h}")
        check_lse(to64(lse[0, h]), lref, f"zero-scale LSE h={h}")
