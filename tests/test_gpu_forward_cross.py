"""GPU parity of fa_forward_cross (Nq query rows against Nk keys) with the fp64 oracle.

The oracle is `oracle.attention.decode`, whose rows are the last Nq positions of
the sequence of Nk keys (under the causal mask row i sees keys 0 .. Nk - Nq + i;
without it the positions do not matter).  Bars as for the forward.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.attention as ora
import synth
from gpu_helpers import check, check_lse, require_gpu, say, to_dev, to64

pytestmark = pytest.mark.gpu

CASES = [
    # B, Nq, Nk, H, d, causal
    (1, 100, 300, 2, 64, True),
    (2, 257, 1000, 2, 128, True),
    (1, 64, 64, 2, 64, True),          # Nq = Nk: the square forward
    (1, 500, 200, 2, 64, False),       # more query rows than keys
    (1, 1, 4096, 2, 128, True),
    (2, 129, 4097, 3, 64, False),
    (1, 384, 5000, 2, 128, False),
    (1, 1000, 1001, 1, 64, True),
]


@pytest.mark.parametrize("B,Nq,Nk,H,d,causal", CASES)
def test_forward_cross_matches_oracle(B, Nq, Nk, H, d, causal):
    require_gpu()
    say("forward_cross", B, Nq, Nk, H, d, causal)
    host = synth.make_decode_inputs(B, Nq, Nk, H, d, seed=2000 + Nq + Nk)
    q, k, v = (to_dev(host[x]) for x in "qkv")
    f64 = {x: synth.decode(host[x]) for x in "qkv"}
    scale = synth.f32(d ** -0.5)
    o, lse = fa.forward_cross(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o64, lse64 = to64(o), to64(lse)
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = ora.decode(f64["q"][b, :, h], f64["k"][b, :, h], f64["v"][b, :, h], scale, causal)
            check(o64[b, :, h], o_ref, "bf16", f"cross O (b={b}, h={h})")
            check_lse(lse64[b, h], lse_ref, f"cross LSE (b={b}, h={h})")


def test_forward_cross_square_is_bitwise_forward():
    """With Nq = Nk the entry point runs the same kernel as fa_forward."""
    require_gpu()
    for d, causal in ((64, True), (128, True), (128, False)):
        host = synth.make_decode_inputs(2, 300, 300, 2, d, seed=31)
        q, k, v = (to_dev(host[x]) for x in "qkv")
        o1, l1 = fa.forward(q, k, v, causal=causal)
        o2, l2 = fa.forward_cross(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
