"""Head size 256 (bf16): forward, backward and the cross-length entry points
against the fp64 oracle, under the same bars as d = 64 and 128."""
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.attention as ora
import synth
from gpu_helpers import check, check_lse, inputs, require_gpu, say, to_dev, to64
from test_gpu_backward import run_and_check as run_backward
from test_gpu_forward import run_and_check as run_forward

pytestmark = pytest.mark.gpu

D = 256


@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_ragged(N, causal):
    require_gpu()
    run_forward((2, N, 2, D), "bf16", 6000 + N, causal, D ** -0.5, tag="d256")


@pytest.mark.parametrize("N", [1, 17, 100, 129, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged(N, causal):
    require_gpu()
    run_backward((2, N, 2, D), "bf16", 6100 + N, causal, D ** -0.5, tag="d256")


@pytest.mark.parametrize("causal", [False, True])
def test_head_groups(causal):
    """B*H a multiple of 8 with a ragged last tile."""
    require_gpu()
    run_backward((2, 300, 4, D), "bf16", 6200, causal, D ** -0.5, tag="d256 groups")


@pytest.mark.parametrize("causal", [False, True])
def test_midsize(causal):
    require_gpu()
    run_forward((1, 2048, 4, D), "bf16", 6300, causal, D ** -0.5, heads=[(0, 0), (0, 3)], tag="d256 mid")
    run_backward((1, 2048, 4, D), "bf16", 6301, causal, D ** -0.5, heads=[(0, 1), (0, 2)], tag="d256 mid")


@pytest.mark.parametrize("shape", [(2, 4096, 16, D), (1, 4000, 32, D)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_forward_wide_grid(shape, causal):
    """Grids of at least 512 workgroups of 256 rows take the 8-wave form of the
    d = 256 forward (ragged last tile in the second shape)."""
    require_gpu()
    B, N, H, _ = shape
    run_forward(shape, "bf16", 6500 + N, causal, D ** -0.5, heads=[(0, 0), (B - 1, H - 1)], tag="d256 wide")


def test_cross_forward_wide_grid():
    """Nq rows against Nk keys with 512 workgroups of 256 rows: the 8-wave form
    with a query offset under the mask."""
    require_gpu()
    B, Nq, Nk, H = 1, 2000, 3000, 64
    say("d256 wide cross", B, Nq, Nk, H)
    host = synth.make_decode_inputs(B, Nq, Nk, H, D, seed=6600)
    q, k, v = (to_dev(host[x]) for x in "qkv")
    f64 = {x: synth.decode(host[x]) for x in "qkv"}
    scale = synth.f32(D ** -0.5)
    o, lse = fa.forward_cross(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        o_ref, lse_ref = ora.decode(f64["q"][0, :, h], f64["k"][0, :, h], f64["v"][0, :, h], scale, True)
        check(to64(o[0, :, h]), o_ref, "bf16", f"d256 wide cross O h={h}")
        check_lse(to64(lse[0, h]), lse_ref, f"d256 wide cross LSE h={h}")


@pytest.mark.parametrize("B,Nq,Nk,H,causal", [(1, 100, 300, 2, True), (1, 257, 1000, 2, False),
                                             (2, 64, 65, 1, True)])
def test_cross_forward_and_backward(B, Nq, Nk, H, causal):
    require_gpu()
    say("d256 cross", B, Nq, Nk, H, causal)
    host = synth.make_decode_inputs(B, Nq, Nk, H, D, seed=6400 + Nq + Nk, with_do=True)
    q, k, v, do = (to_dev(host[x]) for x in ("q", "k", "v", "do"))
    f64 = {x: synth.decode(host[x]) for x in ("q", "k", "v", "do")}
    scale = synth.f32(D ** -0.5)
    o, lse = fa.forward_cross(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_cross(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = (f64[x][b, :, h] for x in ("q", "k", "v", "do"))
            o_ref, lse_ref = ora.decode(qh, kh, vh, scale, causal)
            check(to64(o[b, :, h]), o_ref, "bf16", f"d256 cross O b={b} h={h}")
            check_lse(to64(lse[b, h]), lse_ref, f"d256 cross LSE b={b} h={h}")
            dq_r, dk_r, dv_r, _ = ora.backward_cross(qh, kh, vh, doh, scale, causal)
            for name, got, ref in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
                check(to64(got[b, :, h]), ref, "bf16", f"d256 cross {name} b={b} h={h}")


@pytest.mark.parametrize("shape", [(2, 300, 3, D), (1, 700, 2, D)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_separate_passes(shape, causal):
    """fa_backward_preprocess, fa_backward_dkdv and fa_backward_dq launched
    apart (at this head size eight-wave workgroups whose wave pairs share
    rows: dQ by a score wave and a dQ wave; dK/dV by role pairs without the
    mask and by column-split pairs under it) against the oracle.
    fa_backward runs the same tiles as one grid and gives the same bits."""
    require_gpu()
    fa_ = fa
    B, N, H, d = shape
    scale = d ** -0.5
    say(f"d256 separate passes shape={shape} causal={causal}")
    dev, f64 = inputs(shape, "bf16", 6500 + N, with_do=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = fa_.forward(q, k, v, scale=scale, causal=causal)
    ws = torch.empty(fa_.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_.fa_backward_preprocess(o, do, lse, ws)
    fa_.fa_backward_dkdv(q, k, v, do, ws, dk, dv, scale, causal)
    fa_.fa_backward_dq(q, k, v, do, ws, dq, scale, causal)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = (f64[x][b, :, h] for x in ("q", "k", "v", "do"))
            dq_r, dk_r, dv_r, _ = ora.backward(qh, kh, vh, doh, scale, causal)
            for name, got, ref in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
                check(to64(got[b, :, h]), ref, "bf16", f"d256 separate {name} b={b} h={h}")
    fused = fa_.backward(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for name, a, b_ in zip(("dQ", "dK", "dV"), (dq, dk, dv), fused):
        assert torch.equal(a, b_), f"{name}: separate passes and fa_backward differ"
    say("  ok")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_repeats_bitwise(causal):
    """The eight-wave pair tiles hand scores or probabilities from one wave to
    its partner through LDS and copy tiles one or two steps ahead: four calls
    of fa_backward on the same inputs give the same bits (a missing wait would
    let a read see a slot's previous contents in some calls and not others)."""
    require_gpu()
    shape = (2, 1000, 4, D)
    say(f"d256 backward repeats shape={shape} causal={causal}")
    dev, _ = inputs(shape, "bf16", 6700, with_do=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = fa.forward(q, k, v, causal=causal)
    first = fa.backward(q, k, v, o, do, lse, causal=causal)
    for _ in range(3):
        again = fa.backward(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), first, again):
            assert torch.equal(a, b), f"{name}: fa_backward gave different bits on a repeated call"
    say("  ok")


@pytest.mark.parametrize("causal", [True, False])
def test_backward_bench_shape_sampled_heads(causal):
    """The bench's d = 256 workload, [2, 4096, 16, 256], in the launch
    configuration it times (fa_forward + fa_backward: eight-wave pair tiles
    over 2048 workgroups); two heads checked element by element against the
    oracle (each an fp64 4096 x 4096 problem)."""
    require_gpu()
    heads = [(0, 0), (1, 15)] if causal else [(1, 7)]
    run_backward((2, 4096, 16, D), "bf16", 6800, causal, D ** -0.5, heads=heads, tag="d256 bench shape")


@pytest.mark.parametrize("causal", [True, False])
def test_forward_bench_shape_sampled_heads(causal):
    """The bench's d = 256 forward, [2, 4096, 16, 256], in the launch
    configuration it times (the 8-wave form over 512 workgroups; under the
    mask with the eager reference max), two heads against the oracle."""
    require_gpu()
    run_forward((2, 4096, 16, D), "bf16", 6900, causal, D ** -0.5, heads=[(0, 3), (1, 12)], tag="d256 bench shape")
