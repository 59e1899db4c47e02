"""Error bounds for the FP8 forward's parity tests (test helper, CPU only).

The GPU result is gated on one oracle of oracle/fp8.py, forward(): the exact
attention of the dequantised inputs.  Every row must lie within `loose_bound`,
the sum of
  - the e4m3 rounding of y = 2^8 p (OCP E4M3: 3 mantissa bits, so round to
    nearest moves a normal y by at most 2^-4 y, a subnormal one by at most
    half the spacing 2^-9, i.e. 2^-10): |round(y) - y| <= max(2^-4 y, 2^-10)
    for 0 <= y <= 448, so O moves by at most
    dv sum_j max(2^-4 2^8 p_ij, 2^-10) |V_jc| / (2^8 l_i); this holds
    whatever maximum the kernel took p against (a smaller maximum only makes
    y larger and the relative bound tighter).  The conversion instruction
    (v_cvt_pk_fp8_f32) is the round-to-nearest-even form in AMD's ISA
    description (its stochastic-rounding sibling is a separate instruction);
  - the score error of the FP8 matrix product, E_ij (below), which moves
    p_ij by a factor within exp(+-(E_ij + max_j E_ij));
  - the accumulation error of the P V products, EPS_ACC times the sum of
    |Pq V| over all of them;
  - the rounding of O to bf16 (2^-8 relative, with margin).

Accumulator width.  AMD's description of v_mfma_f32_32x32x64_f8f6f4 gives an
fp32 result but not the precision of the internal sum of the 64 products of
one instruction.  Assumed here: every addition inside the instruction keeps at
least ACC_BITS = 16 significant bits (any rounding direction).  Products of
two e4m3 values have at most 8 significant bits and are exact; 63 additions
of relative error at most 2^(1 - 16) give at most 63 2^-15 sum |a_i b_i| per
instruction (first order; the factor 1.01 covers the higher-order terms), and
adding each instruction's sum to the fp32 accumulator at most 2^-24 of the
sum of magnitudes so far per instruction.  tests/test_oracle_fp8.py checks on
the CPU that a model of such a kernel (oracle/fp8.py
forward_narrow_accumulator, 16 bits, truncating) stays within these bounds,
and that a narrower accumulator does not.

`tight_bound` compares against forward_quantised_p_online with the kernel's
64-key blocks (the same rounding decisions as the kernel when the scores are
exact); it is reported as a diagnostic only and gates nothing.
"""
from __future__ import annotations

import numpy as np

import oracle.fp8 as fp8

ACC_BITS = 16                                  # assumed, see above
EPS_INSTR = 1.01 * 63 * 2.0 ** (1 - ACC_BITS)  # one 64-product instruction
KBLK = 64                                      # products per instruction
BF16_REL = 2.0 ** -8
F32_REL = 2.0 ** -20
F32_REL_ACC = 2.0 ** -24
LSE_REL = 1e-5


def _visible(nq, nk, causal):
    rows = np.arange(nk - nq, nk)
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    return np.arange(nk)[None, :] <= rows[:, None]


def eps_acc(n):
    """Relative bound (against the sum of |products|) on the accumulated error
    of an n-term product sum taken KBLK terms per instruction."""
    ninstr = max(1, -(-int(n) // KBLK))
    return EPS_INSTR + ninstr * F32_REL_ACC


def score_error(q8, k8, dq, dk, scale):
    """E_ij: bound on |S_kernel - S_exact| in natural-log units ([nq, nk]):
    the accumulation bound over the d products of a score, plus the float32
    multiply by scale * dq * dk."""
    qa = np.abs(fp8.decode_e4m3(q8))
    ka = np.abs(fp8.decode_e4m3(k8))
    d = q8.shape[1]
    mag = (qa @ ka.T) * float(dq) * float(dk) * float(scale)
    return (eps_acc(d) + 2 * F32_REL_ACC) * mag


def exact_probs(q8, k8, dq, dk, scale, causal):
    q = fp8.decode_e4m3(q8) * float(dq)
    k = fp8.decode_e4m3(k8) * float(dk)
    nq, nk = q.shape[0], k.shape[0]
    s = float(scale) * (q @ k.T)
    vis = _visible(nq, nk, causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    return np.where(vis, np.exp(s - m), 0.0), vis


def loose_bound(q8, k8, v8, descales, scale, causal, o_exact):
    dq, dk, dv = descales
    p, vis = exact_probs(q8, k8, dq, dk, scale, causal)
    l = p.sum(axis=1, keepdims=True)
    va = np.abs(fp8.decode_e4m3(v8))
    e = score_error(q8, k8, dq, dk, scale)
    emax = np.where(vis, e, 0.0).max(axis=1, keepdims=True)
    y = 256.0 * p
    rnd = np.where(vis, np.maximum(2.0 ** -4 * y, 2.0 ** -10), 0.0) / 256.0
    shift = np.expm1(np.where(vis, e, 0.0) + emax + F32_REL)     # relative change of p_ij
    pv = p * (1.0 + shift) + rnd                                   # bound on the kernel's |Pq| / 2^8
    acc = eps_acc(k8.shape[0]) * (pv @ va)
    bound = float(dv) * ((rnd + p * shift) @ va + acc) / l
    # the normaliser l of the kernel moves by at most the largest relative shift
    bound += (2 * (emax + F32_REL) + BF16_REL) * (np.abs(o_exact) + bound)
    return bound


def tight_bound(q8, k8, v8, descales, scale, causal, o_online, aux):
    """Diagnostic only: bound on |O_kernel - O_online| (forward_quantised_p_online
    with 64-key blocks, the kernel's tile) for integer-coded Q and K, whose
    scores an accumulator of ACC_BITS >= 15 bits sums exactly (integer products
    <= 225, sums below 2^15); returns (bound, number of ambiguous p)."""
    dq, dk, dv = descales
    vis = _visible(q8.shape[0], k8.shape[0], causal)
    e = np.zeros(vis.shape)
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
    bound = eps_acc(k8.shape[0]) * a + float(dv) * ((w * spacing) @ va) / l
    bound += (delta.max(axis=1, keepdims=True) + BF16_REL) * (np.abs(o_online) + bound)
    return bound, int(amb.sum())


def lse_bound(q8, k8, descales, scale, causal, lse_exact):
    dq, dk, _ = descales
    vis = _visible(q8.shape[0], k8.shape[0], causal)
    e = np.where(vis, score_error(q8, k8, dq, dk, scale), 0.0)
    return 2 * e.max(axis=1) + LSE_REL * np.maximum(1.0, np.abs(lse_exact))
