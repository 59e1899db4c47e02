"""Error bounds for the FP8 forward's parity tests (test helper, CPU only).

The GPU result is compared with two oracles of oracle/fp8.py:

* forward(): exact attention of the dequantised inputs.  Every row must lie
  within `loose_bound`, the sum of
    - the e4m3 rounding of y = 2^8 p: |round(y) - y| <= max(2^-4 y, 2^-10)
      for 0 <= y <= 448, so O moves by at most
      dv sum_j max(2^-4 2^8 p_ij, 2^-10) |V_jc| / (2^8 l_i); this holds
      whatever maximum the kernel took p against (a smaller maximum only makes
      y larger and the relative bound tighter);
    - the score error of the FP8 matrix product, E_ij (below), which moves
      p_ij by a factor within exp(+-(E_ij + max_j E_ij));
    - the accumulation error of the P V products, EPS_MFMA times the sum of
      |Pq V| over all of them;
    - the rounding of O to bf16 (2^-8 relative, with margin).
* forward_quantised_p_online() with 64-key blocks: the kernel's tiles, met in
  the same order, with p rounded against the same running maximum.  When the
  scores are exact (integer-coded Q and K, below) the kernel and this oracle
  differ only where float32 arithmetic puts 2^8 p on the other side of a
  rounding midpoint.  `tight_bound` allows, for every p whose band
  2^8 p (1 +- delta_ij) holds a midpoint, one e4m3 spacing of |V_jc| (scaled
  by the rescale the block's sum got later), plus the P V accumulation and
  bf16 terms and the normaliser's relative error.

EPS_MFMA bounds the error of the 32x32x64 e4m3 MFMA relative to the sum of
the absolute values of its products.  The hardware's accumulation is narrower
than fp32; the value is measured, not documented: on MI355X, random operands
gave at most 2^-14.9 (standard normal), 2^-12.7 (probability-like B operand)
and 2^-11.5 (operands spread over 2^16) for one product, and chains of 4, 16
and 64 products into one accumulator 2^-14.3, 2^-15.4 and 2^-16.3 of the sum
over the chain (the error does not grow with the chain); 2^-10 is used.
Integer operands of magnitude <= 15 (products and sums of up to 128 products
exact in a narrow accumulator) gave no error at all, for one and two chained
products.
"""
from __future__ import annotations

import numpy as np

import oracle.fp8 as fp8

EPS_MFMA = 2.0 ** -10
BF16_REL = 2.0 ** -8
F32_REL = 2.0 ** -20
LSE_REL = 1e-5


def _visible(nq, nk, causal):
    rows = np.arange(nk - nq, nk)
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    return np.arange(nk)[None, :] <= rows[:, None]


def score_error(q8, k8, dq, dk, scale, exact=False):
    """E_ij: bound on |S_kernel - S_exact| in natural-log units ([nq, nk]).

    exact=True: Q and K codes are integers of magnitude <= 15, so every
    product is an integer <= 225 and a score is an integer sum below 2^15;
    such products and sums came out exact on MI355X (measured), E = 0."""
    if exact:
        return np.zeros((q8.shape[0], k8.shape[0]))
    qa = np.abs(fp8.decode_e4m3(q8))
    ka = np.abs(fp8.decode_e4m3(k8))
    d = q8.shape[1]
    # one MFMA per 64 of d, each adding its products to the partial sum
    nprod = max(1, d // 64)
    return nprod * EPS_MFMA * (qa @ ka.T) * float(dq) * float(dk) * float(scale)


def exact_probs(q8, k8, dq, dk, scale, causal):
    q = fp8.decode_e4m3(q8) * float(dq)
    k = fp8.decode_e4m3(k8) * float(dk)
    nq, nk = q.shape[0], k.shape[0]
    s = float(scale) * (q @ k.T)
    vis = _visible(nq, nk, causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    return np.where(vis, np.exp(s - m), 0.0), vis


def loose_bound(q8, k8, v8, descales, scale, causal, o_exact, exact_scores=False):
    dq, dk, dv = descales
    p, vis = exact_probs(q8, k8, dq, dk, scale, causal)
    l = p.sum(axis=1, keepdims=True)
    va = np.abs(fp8.decode_e4m3(v8))
    e = score_error(q8, k8, dq, dk, scale, exact_scores)
    emax = np.where(vis, e, 0.0).max(axis=1, keepdims=True)
    y = 256.0 * p
    rnd = np.where(vis, np.maximum(2.0 ** -4 * y, 2.0 ** -10), 0.0) / 256.0
    shift = np.expm1(np.where(vis, e, 0.0) + emax + F32_REL)     # relative change of p_ij
    pv = p * (1.0 + shift) + rnd                                   # bound on the kernel's |Pq| / 2^8
    acc = EPS_MFMA * (pv @ va)
    bound = float(dv) * ((rnd + p * shift) @ va + acc) / l
    # the normaliser l of the kernel moves by at most the largest relative shift
    bound += (2 * (emax + F32_REL) + BF16_REL) * (np.abs(o_exact) + bound)
    return bound


def tight_bound(q8, k8, v8, descales, scale, causal, o_online, aux, exact_scores=True):
    """Bound on |O_kernel - O_online| (forward_quantised_p_online with 64-key
    blocks, the kernel's tile); returns (bound, number of ambiguous p)."""
    dq, dk, dv = descales
    vis = _visible(q8.shape[0], k8.shape[0], causal)
    e = np.where(vis, score_error(q8, k8, dq, dk, scale, exact_scores), 0.0)
    emax = e.max(axis=1, keepdims=True)
    x = np.where(vis, aux["x"].astype(np.float64), 0.0)
    delta = e + emax + F32_REL * (2.0 + 2.0 * np.abs(x))
    y = 256.0 * aux["p"].astype(np.float64)
    lo = fp8.round_e4m3(y * (1.0 - delta))
    hi = fp8.round_e4m3(y * (1.0 + delta))
    amb = vis & (lo != hi)
    spacing = np.where(amb, np.maximum(hi - lo, fp8.e4m3_spacing(hi)), 0.0)
    # each rounded value reaches O scaled by exp(m_b - m): its block's maximum
    # against the final one
    mref, m = aux["mref"], aux["m"][:, None]
    w = np.where(vis & np.isfinite(mref), np.exp(np.where(np.isfinite(mref), mref - m, 0.0)), 0.0)
    va = np.abs(fp8.decode_e4m3(v8))
    l = 256.0 * aux["l"][:, None]
    a = ((w * aux["pq"]) @ va) * float(dv) / l
    bound = EPS_MFMA * a + float(dv) * ((w * spacing) @ va) / l
    bound += (delta.max(axis=1, keepdims=True) + BF16_REL) * (np.abs(o_online) + bound)
    return bound, int(amb.sum())


def lse_bound(q8, k8, descales, scale, causal, lse_exact, exact_scores=False):
    dq, dk, _ = descales
    vis = _visible(q8.shape[0], k8.shape[0], causal)
    e = np.where(vis, score_error(q8, k8, dq, dk, scale, exact_scores), 0.0)
    return 2 * e.max(axis=1) + LSE_REL * np.maximum(1.0, np.abs(lse_exact))
