"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU path never calls it and shares no code
with it.  It materialises the full score matrix S and probability matrix P, in
float64, with no tiling and no online recurrence: it is the definition the fused
kernels must reproduce up to rounding order.

Sources (pages, with the part of each page followed):
  [FAN] page "FlashAttention" (vagrantpi.github.io PKM note), part "標準 attention
        在幹嘛（IO 的角度）": S = QK^T/sqrt(d), P = softmax(S), O = PV; and "三招"
        item 3 (Recomputation): the forward keeps O and the per-row softmax
        statistics, the backward rebuilds P from them.
  [XH]  page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org):
        section 2 (standard attention formula softmax(QK^T/sqrt(d_k))V),
        section 4 (numerically safe softmax: subtract the row maximum),
        the function standard_attention under "标准注意力对比" (scale, then a
        causal mask that sets entries above the diagonal to -inf, then a row
        softmax, then the product with V), and section 6 (backward).
  [GWL] page "Flash Attention 到底做了什么？" (guanweilu.cn), section
        "它不是一个近似算法": the fused method equals the plain computation except
        for floating-point rounding order, so the plain computation is the oracle.
  [FAN] part "⚠️ 注意": in decode each step has a single query token against
        the KV cache, and the variant for that case is FlashDecoding; part
        "三招" item 2 (online softmax): partial softmax results over disjoint
        key blocks combine by rescaling with exp(m_part - m_total).

Readings taken where the pages are silent or garbled:
  * The saved statistics are the natural-log logsumexp LSE_i = m_i + ln(l_i) per
    query row (the pages save the pair (m, l); LSE carries the same information).
  * The causal mask hides key j from query i when j > i, by absolute index
    (standard_attention's triu(diagonal=1) over the full matrix).
  * The backward formula printed in [XH] section 6 is garbled; the oracle uses
    the chain rule of softmax: dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij,
    dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
  * A row whose keys are all masked has no softmax; it is defined as O = 0 and
    LSE = -inf (this cannot happen for square causal attention).
  * Decode: the nq query rows are the last nq positions of a sequence of nk
    keys, so under the causal mask row i sees keys 0 .. nk - nq + i.  The
    backward of such rows (backward_cross) is the same chain rule over that
    masked score matrix.  The pages
    give no more detail of FlashDecoding than its name; the reading taken is
    the plainest one that the online softmax supports: the keys are split into
    chunks, each chunk gives a normalised partial output and its LSE, and the
    partials combine as LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores", "softmax_rows", "forward", "forward_rows", "backward",
    "decode", "merge_partials", "backward_cross",
]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale, causal, rows=None):
    """S = scale * q k^T with the causal mask applied ([XH] standard_attention).

    q: [nq, d] query rows; k: [nk, d]; rows: absolute query index of each q row
    (default 0..nq-1).  Masked entries are -inf.
    """
    q, k = _as64(q), _as64(k)
    s = float(scale) * (q @ k.T)
    if causal:
        qi = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        hidden = np.arange(k.shape[0])[None, :] > qi[:, None]
        s = np.where(hidden, -np.inf, s)
    return s


def softmax_rows(s):
    """Row softmax with the row maximum subtracted first ([XH] section 4).

    Returns (P, m, l, lse): P = exp(S - m) / l, m the row max, l the row sum of
    exp(S - m), lse = m + ln l.  Fully masked rows give P = 0, lse = -inf.
    """
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked entries
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return p, m, l, lse


def forward(q, k, v, scale, causal):
    """One head: O = softmax(scale q k^T [+mask]) v and the per-row LSE."""
    p, _, _, lse = softmax_rows(scores(q, k, scale, causal))
    return p @ _as64(v), lse


def forward_rows(q_rows, rows, k, v, scale, causal):
    """O and LSE for a subset of query rows (absolute indices `rows`) of one head."""
    p, _, _, lse = softmax_rows(scores(q_rows, k, scale, causal, rows=rows))
    return p @ _as64(v), lse


def decode(q, k, v, scale, causal):
    """Decode against a KV cache ([FAN] "⚠️ 注意"): the nq rows of q are the last
    nq positions of the sequence of len(k) keys; O and LSE of those rows."""
    nq, nk = np.shape(q)[0], np.shape(k)[0]
    return forward_rows(q, np.arange(nk - nq, nk), k, v, scale, causal)


def merge_partials(o_parts, lse_parts):
    """Combine normalised partial results of disjoint key chunks ([FAN] "三招"
    item 2 applied to whole chunks): LSE = log sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s.  o_parts: [S, nq, d]; lse_parts: [S, nq],
    -inf for a chunk in which a row sees no key.  A row with no key in any chunk
    gets O = 0 and LSE = -inf."""
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None, :])            # exp(-inf) = 0
    tot = w.sum(axis=0)
    tot_safe = np.where(empty, 1.0, tot)
    o = (w[:, :, None] * o_parts).sum(axis=0) / tot_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))
    return np.where(empty[:, None], 0.0, o), lse


def backward(q, k, v, do, scale, causal, rows=None):
    """One head: (dQ, dK, dV) of the loss sum(O * dO), by the chain rule.

    rows: absolute query index of each q row, as in :func:`scores` (default
    0..nq-1).  Also returns D_i = sum_j P_ij dP_ij, which equals rowsum(dO * O).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    p, _, _, _ = softmax_rows(scores(q, k, scale, causal, rows=rows))
    dv = p.T @ do
    dp = do @ v.T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv, dvec


def backward_cross(q, k, v, do, scale, causal):
    """Backward of :func:`decode` (nq query rows against len(k) keys, the rows
    being the last nq positions of the sequence): (dQ, dK, dV, D)."""
    nq, nk = np.shape(q)[0], np.shape(k)[0]
    return backward(q, k, v, do, scale, causal, rows=np.arange(nk - nq, nk))
