"""Checks that pin the CPU oracle to facts other than itself.

Each pin takes the oracle module (or a copy with a planted mistake) and raises
AssertionError when the implementation disagrees with a closed form, an
invariant, a library routine or a numerical derivative.  Sources:

  * Q = 0 makes every score equal, so each row of P is uniform: O is the row
    mean of V and LSE = ln(number of visible keys).
  * Softmax rows sum to one, so V = 1 gives O = 1.
  * Without a mask the result does not depend on the order of the keys when K
    and V rows are permuted together.
  * One dominant logit: O is a two-term weighted mean in closed form.
  * Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = S_00.
  * Causal row i equals unmasked attention over keys 0..i (the mask of
    standard_attention on the page "知识点13 | FlashAttention深度攻略").
  * LSE and P agree with scipy.special.logsumexp / softmax on small inputs.
  * The gradients agree with central finite differences of sum(O * dO), and
    satisfy sum_j dK_j = 0, sum_j dV_j = sum_i dO_i and D = rowsum(dO * O).
  * The worked rescale example of the page "Flash Attention 到底做了什么？"
    (guanweilu.cn) has the closed form l = e^-5 (1 + e^-10 + e^-20) + 1.
  * The backward of rows that are the last positions of a sequence agrees with
    central finite differences of sum(decode(q, k, v) * dO), and with the
    square backward of the whole sequence whose other rows have dO = 0.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def pin_zero_query(ora):
    rng = _rng(11)
    n, d = 23, 8
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    q = np.zeros((n, d))
    o, lse = ora.forward(q, k, v, 0.3, False)
    _close(o, np.tile(v.mean(axis=0), (n, 1)), 1e-13, "Q=0 non-causal O")
    _close(lse, np.full(n, math.log(n)), 1e-13, "Q=0 non-causal LSE")
    o, lse = ora.forward(q, k, v, 0.3, True)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    _close(o, prefix_mean, 1e-13, "Q=0 causal O")
    _close(lse, np.log(np.arange(1, n + 1)), 1e-13, "Q=0 causal LSE")


def pin_unit_values(ora):
    rng = _rng(12)
    n, d = 19, 6
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    for causal in (False, True):
        o, _ = ora.forward(q, k, np.ones((n, d)), 0.7, causal)
        _close(o, np.ones((n, d)), 1e-14, f"V=1 causal={causal}")
        p, _, _, _ = ora.softmax_rows(ora.scores(q, k, 0.7, causal))
        _close(p.sum(axis=1), np.ones(n), 1e-14, "softmax row sums")


def pin_permutation(ora):
    rng = _rng(13)
    n, d = 17, 5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o1, l1 = ora.forward(q, k, v, 0.5, False)
    o2, l2 = ora.forward(q, k[perm], v[perm], 0.5, False)
    _close(o1, o2, 1e-13, "joint K/V permutation O")
    _close(l1, l2, 1e-13, "joint K/V permutation LSE")


def pin_dominant_logit(ora):
    rng = _rng(14)
    n, d, jstar = 29, 4, 7
    scale = 0.125
    a = math.sqrt(50.0 / scale)                 # scale * a^2 = 50
    q = np.zeros((n, d)); q[:, 0] = a
    k = np.zeros((n, d)); k[jstar, 0] = a
    v = rng.standard_normal((n, d))
    o, lse = ora.forward(q, k, v, scale, False)
    w = math.exp(50.0)
    expect = (w * v[jstar] + (v.sum(axis=0) - v[jstar])) / (w + n - 1)
    _close(o, np.tile(expect, (n, 1)), 1e-12, "dominant logit O")
    _close(lse, np.full(n, math.log(w + n - 1)), 1e-12, "dominant logit LSE")


def pin_causal_rows(ora):
    rng = _rng(15)
    n, d, scale = 21, 7, 0.4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = ora.forward(q, k, v, scale, True)
    _close(o[0], v[0], 1e-14, "causal row 0 O")
    _close(lse[0], scale * float(q[0] @ k[0]), 1e-14, "causal row 0 LSE")
    for i in (1, 5, n - 1):
        oi, li = ora.forward(q[i:i + 1], k[:i + 1], v[:i + 1], scale, False)
        _close(o[i], oi[0], 1e-13, f"causal row {i} vs unmasked prefix")
        _close(lse[i], li[0], 1e-13, f"causal row {i} LSE vs unmasked prefix")
    rows = np.array([0, 3, 20])
    o_r, lse_r = ora.forward_rows(q[rows], rows, k, v, scale, True)
    _close(o_r, o[rows], 1e-14, "forward_rows O")
    _close(lse_r, lse[rows], 1e-14, "forward_rows LSE")


def pin_scipy(ora):
    rng = _rng(16)
    n, d, scale = 9, 3, 0.9
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    s = scale * np.array([[sum(q[i, c] * k[j, c] for c in range(d)) for j in range(n)] for i in range(n)])
    p, _, _, lse = ora.softmax_rows(ora.scores(q, k, scale, False))
    _close(lse, scipy.special.logsumexp(s, axis=1), 1e-13, "LSE vs scipy logsumexp")
    _close(p, scipy.special.softmax(s, axis=1), 1e-14, "P vs scipy softmax")
    masked = np.where(np.triu(np.ones((n, n), dtype=bool), 1), -np.inf, s)
    p, _, _, lse = ora.softmax_rows(ora.scores(q, k, scale, True))
    _close(lse, scipy.special.logsumexp(masked, axis=1), 1e-13, "causal LSE vs scipy")
    _close(p, scipy.special.softmax(masked, axis=1), 1e-14, "causal P vs scipy")


def _loss(ora, q, k, v, do, scale, causal):
    o, _ = ora.forward(q, k, v, scale, causal)
    return float((o * do).sum())


def pin_finite_differences(ora):
    rng = _rng(17)
    n, d, scale, h = 11, 5, 0.6, 1e-6
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv, _ = ora.backward(q, k, v, do, scale, causal)
        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                key = name[1].lower()
                args_p[key], args_m[key] = xp, xm
                num[idx] = (_loss(ora, args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                            - _loss(ora, args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * h)
            tol = 1e-6 * max(1.0, float(np.abs(num).max()))
            _close(g, num, tol, f"{name} vs central differences (causal={causal})")


def pin_backward_invariants(ora):
    rng = _rng(18)
    n, d, scale = 24, 6, 0.35
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv, dvec = ora.backward(q, k, v, do, scale, causal)
        o, _ = ora.forward(q, k, v, scale, causal)
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, "sum_j dK_j = 0")
        _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, "sum_j dV_j = sum_i dO_i")
        _close(dvec, (do * o).sum(axis=1), 1e-12, "D = rowsum(dO * O)")
    # A single key: every row attends to it with weight one.
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv, _ = ora.backward(q, k[:1], v[:1], do, scale, False)
    _close(dq, np.zeros_like(q), 1e-13, "single key dQ = 0")
    _close(dk, np.zeros((1, d)), 1e-12, "single key dK = 0")
    _close(dv, do.sum(axis=0, keepdims=True), 1e-12, "single key dV = sum dO")


def pin_worked_example(ora):
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    row = np.concatenate([np.asarray(b, dtype=np.float64) for b in g["blocks"]])[None, :]
    _, m, l, lse = ora.softmax_rows(row)
    m_final = g["running_max_after_each_block"][-1]
    e = g["rescale_exponent_at_second_block"]
    l_closed = math.exp(e) * (1 + math.exp(-10) + math.exp(-20)) + 1.0
    _close(m, [m_final], 0.0, "worked example max")
    _close(l, [l_closed], 1e-15, "worked example running sum")
    _close(lse, [m_final + math.log(l_closed)], 1e-13, "worked example LSE")


def pin_decode(ora):
    """Decode rows are the last rows of the full sequence: under the causal mask
    they equal those rows of the square forward; row 0 of the decode block sees
    exactly the keys of its prefix; without the mask the position is irrelevant;
    one key gives O = V[0] and LSE = the single score."""
    rng = _rng(21)
    nk, nq, d, scale = 13, 4, 6, 0.6
    q_full, k, v = (rng.standard_normal((nk, d)) for _ in range(3))
    q = q_full[nk - nq:]
    o_full, lse_full = ora.forward(q_full, k, v, scale, True)
    o_dec, lse_dec = ora.decode(q, k, v, scale, True)
    _close(o_dec, o_full[nk - nq:], 1e-14, "causal decode O vs last rows of the forward")
    _close(lse_dec, lse_full[nk - nq:], 1e-14, "causal decode LSE vs last rows of the forward")
    o_p, lse_p = ora.forward(q[:1], k[:nk - nq + 1], v[:nk - nq + 1], scale, False)
    _close(o_dec[0], o_p[0], 1e-13, "first decode row vs unmasked prefix")
    _close(lse_dec[0], lse_p[0], 1e-13, "first decode row LSE vs unmasked prefix")
    o_nc, lse_nc = ora.decode(q, k, v, scale, False)
    o_f, lse_f = ora.forward(q, k, v, scale, False)
    _close(o_nc, o_f, 1e-14, "unmasked decode O")
    _close(lse_nc, lse_f, 1e-14, "unmasked decode LSE")
    o1, lse1 = ora.decode(q[:1], k[:1], v[:1], scale, True)
    _close(o1[0], v[0], 1e-15, "single key O")
    _close(lse1, [scale * float(q[0] @ k[0])], 1e-14, "single key LSE")


def pin_merge(ora):
    """Partial results of key chunks merge to the whole-row result (the online
    softmax applied to chunks), whatever the chunking and order, including
    chunks in which some rows see no key; two chunks with equal LSE average
    their outputs and add ln 2 to the LSE."""
    rng = _rng(22)
    nk, nq, d, scale = 17, 5, 4, 0.8
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    rows = np.arange(nk - nq, nk)
    s = ora.scores(q, k, scale, True, rows=rows)
    o_ref, lse_ref = ora.decode(q, k, v, scale, True)
    for cuts in ([0, 5, 6, 17], [0, 17], [0, 1, 2, 9, 13, 14, 17]):
        parts = [(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        o_p, lse_p = [], []
        for a, b in parts:
            p_c, _, _, lse_c = ora.softmax_rows(s[:, a:b])
            o_p.append(p_c @ v[a:b])
            lse_p.append(lse_c)
        for order in (slice(None), slice(None, None, -1)):
            o_m, lse_m = ora.merge_partials(np.array(o_p)[order], np.array(lse_p)[order])
            _close(o_m, o_ref, 1e-13, f"merged O, chunks {cuts}")
            _close(lse_m, lse_ref, 1e-13, f"merged LSE, chunks {cuts}")
    o_a, o_b = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    o_m, lse_m = ora.merge_partials(np.array([o_a, o_b]), np.array([[0.3], [0.3]]))
    _close(o_m, (o_a + o_b) / 2, 1e-15, "equal-weight merge O")
    _close(lse_m, [0.3 + math.log(2.0)], 1e-15, "equal-weight merge LSE")


def pin_backward_cross(ora):
    """Gradients of the last nq rows of a sequence of nk keys."""
    rng = _rng(23)
    nk, nq, d, scale, h = 9, 4, 5, 0.7, 1e-6
    for causal in (True, False):
        q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
        k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
        dq, dk, dv, dvec = ora.backward_cross(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            o, _ = ora.decode(qq, kk, vv, scale, causal)
            return float((o * do).sum())

        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                a_p = {"q": q, "k": k, "v": v}
                a_m = dict(a_p)
                a_p[name[1].lower()], a_m[name[1].lower()] = xp, xm
                num[idx] = (loss(a_p["q"], a_p["k"], a_p["v"]) - loss(a_m["q"], a_m["k"], a_m["v"])) / (2 * h)
            tol = 1e-6 * max(1.0, float(np.abs(num).max()))
            _close(g, num, tol, f"cross {name} vs central differences (causal={causal})")
        o, _ = ora.decode(q, k, v, scale, causal)
        _close(dvec, (do * o).sum(axis=1), 1e-12, "cross D = rowsum(dO * O)")
    # The square backward over the whole sequence with dO = 0 on the first
    # nk - nq rows: those rows contribute nothing to dK and dV.
    q_full, k, v = (rng.standard_normal((nk, d)) for _ in range(3))
    do_full = np.zeros((nk, d))
    do_full[nk - nq:] = rng.standard_normal((nq, d))
    dq_f, dk_f, dv_f, _ = ora.backward(q_full, k, v, do_full, scale, True)
    dq_c, dk_c, dv_c, _ = ora.backward_cross(q_full[nk - nq:], k, v, do_full[nk - nq:], scale, True)
    _close(dq_c, dq_f[nk - nq:], 1e-13, "cross dQ vs last rows of the square backward")
    _close(dk_c, dk_f, 1e-13, "cross dK vs square backward")
    _close(dv_c, dv_f, 1e-13, "cross dV vs square backward")


ALL_PINS = [
    pin_zero_query, pin_unit_values, pin_permutation, pin_dominant_logit, pin_causal_rows,
    pin_scipy, pin_finite_differences, pin_backward_invariants, pin_worked_example,
    pin_decode, pin_merge, pin_backward_cross,
]
