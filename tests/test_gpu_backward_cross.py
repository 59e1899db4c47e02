"""GPU parity of fa_backward_cross (Nq query rows against Nk keys) with the fp64 oracle.

The oracle is `oracle.attention.backward_cross`: the rows are the last Nq
positions of the sequence of Nk keys, as for `decode` (under the causal mask
row i sees keys 0 .. Nk - Nq + i; without it the positions do not matter).
The forward is fa_forward_cross, whose O and LSE the backward consumes.  Bars
as for the backward.
"""
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.attention as ora
import synth
from gpu_helpers import check, require_gpu, say, to_dev, to64

pytestmark = pytest.mark.gpu

CASES = [
    # B, Nq, Nk, H, d, causal
    (1, 100, 300, 2, 64, True),
    (2, 257, 1000, 2, 128, True),
    (1, 500, 200, 2, 64, False),       # more query rows than keys
    (1, 1, 2048, 2, 64, True),         # one row against a long cache
    (1, 384, 1500, 2, 128, False),
    (1, 1000, 1001, 1, 64, True),
    (1, 130, 4000, 2, 128, True),
    (2, 33, 95, 3, 64, True),
]


@pytest.mark.parametrize("B,Nq,Nk,H,d,causal", CASES)
def test_backward_cross_matches_oracle(B, Nq, Nk, H, d, causal):
    require_gpu()
    say("backward_cross", B, Nq, Nk, H, d, causal)
    host = synth.make_decode_inputs(B, Nq, Nk, H, d, seed=3000 + Nq + Nk, with_do=True)
    q, k, v, do = (to_dev(host[x]) for x in ("q", "k", "v", "do"))
    f64 = {x: synth.decode(host[x]) for x in ("q", "k", "v", "do")}
    scale = synth.f32(d ** -0.5)
    o, lse = fa.forward_cross(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_cross(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ref = ora.backward_cross(f64["q"][b, :, h], f64["k"][b, :, h], f64["v"][b, :, h],
                                     f64["do"][b, :, h], scale, causal)
            for name, got, r in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
                check(to64(got[b, :, h]), r, "bf16", f"cross {name} (b={b}, h={h})")


def test_backward_cross_square_is_bitwise_backward():
    """With Nq = Nk the entry point runs exactly what fa_backward runs."""
    require_gpu()
    for d, causal in ((64, True), (64, False), (128, True)):
        host = synth.make_decode_inputs(2, 300, 300, 2, d, seed=41, with_do=True)
        q, k, v, do = (to_dev(host[x]) for x in ("q", "k", "v", "do"))
        o, lse = fa.forward(q, k, v, causal=causal)
        g1 = fa.backward(q, k, v, o, do, lse, causal=causal)
        g2 = fa.backward_cross(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(g1, g2))
