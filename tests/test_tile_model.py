"""The blocked online-softmax model against the plain oracle (CPU, fp64).

This carries the intent of test_equivalence on the page "知识点13 |
FlashAttention深度攻略" (the tiled module equals standard_attention to 1e-5 in
fp32 on B=2, N=64, H=4, d=32 with block 32 and a causal mask), in fp64 and for
many tile shapes and orders, including ragged tails and B_r != B_c.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.attention as ora
from oracle import tile_model as tm

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _data(seed, n, d, count=4):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(count)]


def test_equivalence_shape_of_the_page():
    rng = np.random.default_rng(7)
    B, N, H, d = 2, 64, 4, 32
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            o_t, l_t, _ = tm.tiled_forward(q[b, :, h], k[b, :, h], v[b, :, h], d ** -0.5, True, 32, 32)
            o, l = ora.forward(q[b, :, h], k[b, :, h], v[b, :, h], d ** -0.5, True)
            assert np.abs(o_t - o).max() < 1e-12 and np.abs(l_t - l).max() < 1e-12


@pytest.mark.parametrize("n", [1, 5, 37, 64, 100])
@pytest.mark.parametrize("br,bc", [(16, 16), (32, 16), (16, 32), (64, 128), (7, 5)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["ascending", "descending", "diagonal_first"])
def test_tiled_forward_matches_oracle(n, br, bc, causal, order):
    q, k, v = _data(n * 1000 + br * 10 + bc, n, 8, 3)
    o_t, l_t, _ = tm.tiled_forward(q, k, v, 0.37, causal, br, bc, order)
    o, l = ora.forward(q, k, v, 0.37, causal)
    assert np.isfinite(o_t).all() and np.isfinite(l_t).all()
    assert np.abs(o_t - o).max() < 1e-12
    assert np.abs(l_t - l).max() < 1e-12


def test_causal_skips_blocks_above_diagonal():
    q, k, v = _data(3, 256, 4, 3)
    _, _, full = tm.tiled_forward(q, k, v, 0.5, False, 64, 64)
    _, _, causal = tm.tiled_forward(q, k, v, 0.5, True, 64, 64)
    assert full == 16 and causal == 4 * 5 // 2


@pytest.mark.parametrize("n,br,bc", [(48, 16, 16), (37, 8, 16), (64, 32, 16), (33, 16, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_backward_matches_oracle(n, br, bc, causal):
    q, k, v, do = _data(n + br, n, 6)
    o, lse = ora.forward(q, k, v, 0.45, causal)
    dq_t, dk_t, dv_t, d_t = tm.tiled_backward(q, k, v, o, do, lse, 0.45, causal, br, bc)
    dq, dk, dv, dvec = ora.backward(q, k, v, do, 0.45, causal)
    for a, b in ((dq_t, dq), (dk_t, dk), (dv_t, dv), (d_t, dvec)):
        assert np.abs(a - b).max() < 1e-12


def test_worked_rescale_example():
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    m, l, trace = tm.online_softmax_row(g["blocks"])
    assert [t[0] for t in trace] == g["running_max_after_each_block"]
    assert trace[1][1] == pytest.approx(math.exp(g["rescale_exponent_at_second_block"]), rel=1e-15)
    l_closed = math.exp(-5) * (1 + math.exp(-10) + math.exp(-20)) + 1
    assert l == pytest.approx(l_closed, rel=1e-15)
    assert m + math.log(l) == pytest.approx(95 + math.log(l_closed), rel=1e-15)
