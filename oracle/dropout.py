"""CPU oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU path never calls it and shares no code
with it.

Sources: page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org),
section 7 (operator fusion): the softmax step fused into the one kernel
includes the mask and dropout; page "FlashAttention" (vagrantpi.github.io),
"三招" item 3 (recomputation): the backward rebuilds what the forward used
from saved state instead of storing it.  They give no RNG and no formula; the
readings taken:

  * Dropout acts on the normalised probabilities: O = (P * Z) V with
    Z_ij = keep_ij s (s the inverse keep probability below) and P =
    softmax(S) as without dropout (so the row maximum, the row sum and LSE
    do not change).
  * The mask is not stored: it is a function of (head, query row, key,
    seed, offset), replayed by the backward.  The generator is Philox4x32-10
    (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011): a 4 x 32-bit counter, a 2 x 32-bit
    key, ten rounds, each multiplying words 0 and 2 by 0xD2511F53 and
    0xCD9E8D57 (the high halves XOR words 3 and 1 and the round key), the key
    bumped by 0x9E3779B9 and 0xBB67AE85 between rounds.
  * Each generator call yields eight 16-bit fields (field f is the low half
    of word f / 2 for even f, the high half for odd f).  Element (query row
    i, key j) of head bh = b H + h is field f(j) = 4 (floor(j / 8) mod 2) +
    (j mod 4) of Philox((c(j), i, bh, offset), (seed mod 2^32, seed div
    2^32)) with c(j) = 2 floor(j / 16) + (floor(j / 4) mod 2), so one call
    serves keys 16a + 4b + {0, 1, 2, 3, 8, 9, 10, 11} (b in {0, 1}) of one
    row.  It is kept when the field is >= t = round(p 2^16) (at most
    2^16 - 1): p is taken to the nearest multiple of 2^-16, and kept
    probabilities are scaled by 2^16 / (2^16 - t) = 1 / (1 - t 2^-16), the
    inverse of the keep probability, so dropout stays unbiased.
  * The backward is the chain rule with the mask fixed: dV = (P * Z)^T dO,
    dP = (dO V^T) * Z, D_i = sum_j P_ij dP_ij (= rowsum(dO * O)),
    dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention import scores, softmax_rows

__all__ = ["philox4x32_10", "threshold", "keep_scale", "counter_field", "keep_mask", "forward", "backward"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ctr ([..., 4] uint32) under key (k0, k1)."""
    x = [np.asarray(ctr, dtype=np.uint64)[..., i] for i in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * x[0]
        p1 = _M1 * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x = [hi1 ^ x[1] ^ np.uint64(k0), lo1, hi0 ^ x[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return np.stack(x, axis=-1).astype(np.uint32)


def threshold(p):
    """Fields >= this 16-bit integer are kept: round(p 2^16) (ties to even),
    at most 2^16 - 1, for 0 <= p < 1."""
    return min(int(np.round(float(p) * 65536.0)), 65535)


def keep_scale(p):
    """Multiplier of a kept probability: 2^16 / (2^16 - threshold(p))."""
    return 65536.0 / (65536 - threshold(p))


def counter_field(j):
    """(counter word 0, field index) of key j (integer or array)."""
    j = np.asarray(j, dtype=np.uint64)
    c = ((j >> np.uint64(4)) << np.uint64(1)) | ((j >> np.uint64(2)) & np.uint64(1))
    f = (((j >> np.uint64(3)) & np.uint64(1)) << np.uint64(2)) | (j & np.uint64(3))
    return c, f


def keep_mask(bh, rows, nk, p, seed, offset=0):
    """Boolean [len(rows), nk]: which (query row, key) elements of head bh are kept."""
    rows = np.asarray(rows, dtype=np.uint64)
    c, f = counter_field(np.arange(nk))
    ctr = np.zeros((rows.size, nk, 4), dtype=np.uint64)
    ctr[..., 0] = c[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = np.uint64(bh)
    ctr[..., 3] = np.uint64(offset)
    words = philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)).astype(np.uint64)
    idx = (f >> np.uint64(1)).astype(np.int64)[None, :, None].repeat(rows.size, 0)
    word = np.take_along_axis(words, idx, axis=2)[..., 0]
    field = (word >> (np.uint64(16) * (f & np.uint64(1)))[None, :]) & np.uint64(0xFFFF)
    return field >= np.uint64(threshold(p))


def forward(q, k, v, scale, causal, keep, p):
    """O = (P * keep * keep_scale(p)) V and LSE (unchanged by dropout), float64."""
    s = scores(q, k, scale, causal)
    pm, _, _, lse = softmax_rows(s)
    z = np.where(keep, keep_scale(p), 0.0)
    return (pm * z) @ np.asarray(v, dtype=np.float64), lse


def backward(q, k, v, do, scale, causal, keep, p):
    """dQ, dK, dV of sum(O * dO) for forward() with the mask fixed, and D."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    pm, _, _, _ = softmax_rows(scores(q, k, scale, causal))
    z = np.where(keep, keep_scale(p), 0.0)
    dv = (pm * z).T @ do
    dp = (do @ v.T) * z
    dvec = (pm * dp).sum(axis=1)
    ds = pm * (dp - dvec[:, None])
    return float(scale) * ds @ k, float(scale) * ds.T @ q, dv, dvec
