"""fp64 model of the tiled, online-softmax attention algorithm.

TEST INFRASTRUCTURE. It is not the definition (that is oracle.attention); it
spells out, in plain numpy, the blocked algorithm the GPU kernels run, so the
tests can show on the CPU that the recurrence, the causal tile skipping and the
LSE-based recomputation reach the plain result for any tile shape and order.

Sources:
  [FAN] page "FlashAttention" (vagrantpi.github.io PKM note), "三招":
        item 1 (tiling: for each Q block, stream the K/V blocks through on-chip
        memory and write only O), item 2 (online softmax: per row keep a running
        max m, running sum l and an unnormalised output O; for block j,
        m_new = max(m_old, rowmax S_j), P_j = exp(S_j - m_new),
        l_new = exp(m_old - m_new) l_old + rowsum P_j,
        O_new = diag(exp(m_old - m_new)) O_old + P_j V_j, and divide O by l once
        at the end), item 3 (recomputation in the backward from saved statistics).
  [GWL] page "Flash Attention 到底做了什么？" (guanweilu.cn), section
        "分块算出来的 softmax，凭什么和整行算的分毫不差": the worked rescale of a
        block [90, 80, 70] when a later block brings 95.
  [XH]  page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org), section 3
        (Q split into T_r blocks of B_r rows, K and V into T_c blocks of B_c rows)
        and the follow-up on FlashAttention-2 (parallelise over the sequence:
        Q blocks outermost, which keeps m, l and O of a Q block on chip).

Readings: the scale multiplies S before the max and the exponent (the pseudocode
in [XH] section 3 omits it; its module and standard_attention apply it).  The
block output added to O is exp(S_j - m_new) V_j, not a per-block normalised
softmax (the pseudocode's softmax(S_block) @ V_block and the normalised update in
[XH] section 4 disagree with the one-final-divide form of [FAN]).  The causal
mask is by absolute index, so blocks entirely above the diagonal are skipped and
only blocks that straddle it are masked element by element.
"""
from __future__ import annotations

import numpy as np


def _blocks(n, size):
    return [(s, min(s + size, n)) for s in range(0, n, size)]


def _kv_order(kv_blocks, order):
    if order == "ascending":
        return list(kv_blocks)
    if order == "descending":
        return list(reversed(kv_blocks))
    if order == "diagonal_first":          # last (diagonal) block first, then the rest
        return list(kv_blocks[-1:]) + list(kv_blocks[:-1])
    raise ValueError(order)


def online_softmax_row(blocks):
    """The recurrence of [FAN] item 2 on one row of scores given block by block.

    Returns (m, l, trace) where trace lists (m_new, alpha, l_new) after each block.
    """
    m, l, trace = -np.inf, 0.0, []
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.float64)
        m_new = max(m, float(blk.max()))
        alpha = 1.0 if m == -np.inf else float(np.exp(m - m_new))
        l = alpha * l + float(np.exp(blk - m_new).sum())
        m = m_new
        trace.append((m_new, alpha, l))
    return m, l, trace


def tiled_forward(q, k, v, scale, causal, br, bc, order="ascending"):
    """Blocked forward of one head: Q blocks outer, K/V blocks inner.

    Returns (O, LSE, visited) where visited counts the (q-block, kv-block) pairs
    that were computed (causal skips the ones wholly above the diagonal).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    nk = k.shape[0]
    o = np.zeros((n, d))
    lse = np.empty(n)
    visited = 0
    for (r0, r1) in _blocks(n, br):
        kv = _blocks(nk, bc)
        if causal:
            kv = [(c0, c1) for (c0, c1) in kv if c0 <= r1 - 1]   # skip blocks above the diagonal
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, d))
        for (c0, c1) in _kv_order(kv, order):
            visited += 1
            s = scale * (q[r0:r1] @ k[c0:c1].T)
            if causal:
                hidden = np.arange(c0, c1)[None, :] > np.arange(r0, r1)[:, None]
                s = np.where(hidden, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            # A row that has seen only masked keys keeps m = -inf; its factors are
            # defined as alpha = 1 and P = 0 so that no inf - inf appears.
            live = np.isfinite(m_new)
            m_ref = np.where(live, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - m_ref), 1.0)
            p = np.exp(s - m_ref[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[c0:c1]
            m = m_new
        empty = ~np.isfinite(m)
        o[r0:r1] = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, l)[:, None])
        with np.errstate(divide="ignore"):
            lse[r0:r1] = np.where(empty, -np.inf, np.where(empty, 0.0, m) + np.log(np.where(empty, 1.0, l)))
    return o, lse, visited


def tiled_backward(q, k, v, o, do, lse, scale, causal, br, bc):
    """Two-pass blocked backward that rebuilds P from the saved LSE.

    D = rowsum(dO * O); pass 1 holds one K/V block and walks the Q blocks that
    can see it (dK, dV); pass 2 holds one Q block and walks the K/V blocks it can
    see (dQ).  P_ij = exp(scale q_i k_j - LSE_i) is recomputed in both passes.
    """
    q, k, v, o, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    n, d = q.shape
    dvec = (do * o).sum(axis=1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)

    def tile(r0, r1, c0, c1):
        s = scale * (q[r0:r1] @ k[c0:c1].T)
        if causal:
            s = np.where(np.arange(c0, c1)[None, :] > np.arange(r0, r1)[:, None], -np.inf, s)
        p = np.exp(s - lse[r0:r1, None])
        dp = do[r0:r1] @ v[c0:c1].T
        ds = p * (dp - dvec[r0:r1, None])
        return p, ds

    for (c0, c1) in _blocks(n, bc):                       # pass 1: dK, dV
        for (r0, r1) in _blocks(n, br):
            if causal and r1 - 1 < c0:
                continue
            p, ds = tile(r0, r1, c0, c1)
            dv[c0:c1] += p.T @ do[r0:r1]
            dk[c0:c1] += ds.T @ q[r0:r1]
    for (r0, r1) in _blocks(n, br):                       # pass 2: dQ
        for (c0, c1) in _blocks(n, bc):
            if causal and c0 > r1 - 1:
                continue
            _, ds = tile(r0, r1, c0, c1)
            dq[r0:r1] += ds @ k[c0:c1]
    return scale * dq, scale * dk, dv, dvec
