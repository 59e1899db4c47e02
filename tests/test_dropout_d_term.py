"""The dropout bars' D term (gpu_helpers.dropout_d_terms) against the effect it
bounds, on the CPU: the chain rule of the dropout backward with D taken from
the bf16-rounded output O moves dQ and dK by no more than the term, element by
element, and the term is nearly attained where a causal row sees one key."""
import numpy as np
import torch

import oracle.dropout as drop
import synth
from gpu_helpers import dropout_d_terms


def _bf16(x):
    return torch.tensor(np.asarray(x), dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()


def _grads_with_d(q, k, v, do, scale, causal, keep, p, dvec):
    """dQ, dK of dS = P * (Z * (dO V^T) - D) for a given D (the oracle's chain rule)."""
    pm = drop.softmax_rows(drop.scores(q, k, scale, causal))[0]
    z = np.where(keep, drop.keep_scale(p), 0.0)
    ds = pm * ((do @ v.T) * z - dvec[:, None])
    return scale * ds @ k, scale * ds.T @ q


def test_d_term_bounds_the_rounding_of_o():
    # the case of the seeded sweep where the term matters: d = 256, causal, p = 0.35
    N, d, p, seed = 256, 256, 0.3499905895773784, 628500724
    scale = synth.f32(1.5745487861282543 * d ** -0.5)
    host = synth.make_inputs((3, N, 1, d), "bf16", seed, with_do=True)
    q, k, v, do = (synth.decode(host[x])[1, :, 0] for x in ("q", "k", "v", "do"))
    keep = drop.keep_mask(1, np.arange(N), N, p, 5799996125677310176, 111838774)
    o, _ = drop.forward(q, k, v, scale, True, keep, p)
    dq_x, dk_x = _grads_with_d(q, k, v, do, scale, True, keep, p, (do * o).sum(axis=1))
    dq_r, dk_r = _grads_with_d(q, k, v, do, scale, True, keep, p, (do * _bf16(o)).sum(axis=1))
    dq_t, dk_t = dropout_d_terms(q, k, do, o, scale, True)
    for name, a, b, t in (("dQ", dq_x, dq_r, dq_t), ("dK", dk_x, dk_r, dk_t)):
        shift = np.abs(a - b)
        assert (shift <= t).all(), f"{name}: shift {(shift - t).max():.3e} beyond the term"
    # not vacuous: the one-key row 0 moves by a fifth or more of its worst-case
    # bound (which takes every rounding error at its largest, with one sign)
    ratio = (np.abs(dq_x - dq_r)[0] / dq_t[0]).max()
    assert ratio > 0.2, ratio
    # and the exact chain rule with the exact D is the oracle's backward
    ref = drop.backward(q, k, v, do, scale, True, keep, p)
    assert np.allclose(dq_x, ref[0], atol=1e-12) and np.allclose(dk_x, ref[1], atol=1e-12)
