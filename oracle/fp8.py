"""CPU oracle for the FP8 (e4m3) attention forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU path never calls it and shares no code
with it.

Sources (pages, with the part of each page followed):
  [FAN] page "FlashAttention" (vagrantpi.github.io PKM note), part "效果":
        the table row of FlashAttention-3 (FP8 goes beyond its bf16 speed-up)
        and the paragraph under the table (FA3 uses Hopper features, FP8 among
        them).
  [XH]  page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org), part
        "前沿研究方向": mixed precision with low-precision formats such as FP8.
  For e4m3 itself the pages give no definition; the format followed is the
  8-bit floating point E4M3 of the OCP "OFP8" specification: 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits, subnormals when the exponent
  field is 0, no infinities, the two codes S.1111.111 are NaN, and the largest
  finite magnitude is 448.

What is computed (the readings taken, since the pages only name FP8):
  * Q, K and V arrive as e4m3 codes with one fp32 descale factor per tensor
    (dq, dk, dv): the value of an element is decode(code) * descale.
  * forward(): the exact attention of those values, in float64:
        S = scale * dq * dk * Q8 K8^T (causal mask as in the bf16 path),
        P = softmax(S), O = dv * P V8, LSE = m + ln l.
    This is the result the method approximates.
  * forward_quantised_p(): the same, except that the probabilities enter the
    second product as e4m3 codes, which is what lets both products of the
    forward run on FP8 matrix units.  The row maximum is taken first, then
        p_ij = exp(S_ij - m_i)            (float32, as the kernel computes it)
        Pq_ij = round_e4m3(p_scale * p_ij) (round to nearest, ties to even)
        O_i = dv * sum_j Pq_ij V8_j / (p_scale * sum_j p_ij)
    The normaliser uses the unrounded p, so LSE is the same as in forward().
    p_scale = 2^8 puts p in [0, 1] into [0, 256], inside the normal range of
    e4m3 (whose largest value is 448) for every p >= 2^-14; the factor cancels
    in O.  The exponent is formed in float32 from the float64 score rounded to
    float32, so the rounding decisions are taken in the precision the kernel
    takes them in.
  * forward_quantised_p_online(): the same rounding, taken the way the
    online softmax of [FAN] "三招" item 2 meets the keys: block by block
    (blocks of `block` keys, in order, as the B_c-key blocks of [XH] section
    3), each p rounded against the row maximum m_b found so far, the running
    sum and the rounded product rescaled by exp(m_old - m_new) when the
    maximum grows.  It equals forward_quantised_p when every row's maximum
    lies in its first block.  For every row the difference from forward()
    obeys |round_e4m3(y) - y| <= max(2^-4 y, 2^-10) for 0 <= y <= 448,
    whatever maximum p was taken against.
  * round_e4m3 saturates to +-448 (values of p_scale * p never exceed 256).
  * forward_narrow_accumulator(): forward_quantised_p_online computed the way
    a kernel whose FP8 matrix instruction sums its k = 64 products in an
    accumulator of `acc_bits` significant bits would compute it: each block
    of 64 products (64 of d for the scores, 64 keys for P V) is summed in
    order with the running sum truncated toward zero to `acc_bits` bits after
    every addition, and the block's sum is added to a float32 accumulator.
    AMD does not publish the internal width of that accumulator; this model
    of an assumed width lets the tests show on the CPU that their error bound
    covers it.
"""
from __future__ import annotations

import numpy as np

from .attention import scores, softmax_rows

__all__ = ["E4M3_MAX", "decode_e4m3", "round_e4m3", "e4m3_spacing", "truncate_bits",
           "forward", "forward_quantised_p", "forward_quantised_p_online",
           "forward_narrow_accumulator"]

E4M3_MAX = 448.0
_BIAS = 7
_MANT = 3
_EMIN = 1 - _BIAS   # exponent of the smallest normal value, 2^-6


def decode_e4m3(codes):
    """Value of each e4m3 code (uint8 array), float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> _MANT) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - _BIAS)
    sub = np.ldexp(m / 8.0, _EMIN)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_spacing(x):
    """Distance between adjacent e4m3 values around |x| (<= 448).

    2^(e - 3) in the binade [2^e, 2^(e+1)) for e >= -6, and 2^-9 below 2^-6.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, _EMIN)
    return np.ldexp(1.0, (e - _MANT).astype(np.int64))


def round_e4m3(x):
    """Nearest e4m3 value (ties to even mantissa), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    q = e4m3_spacing(x)
    # x / q is exact (q a power of two); np.rint rounds half to even, and an
    # even multiple of the spacing is an even mantissa.  A value that rounds up
    # to the next power of two lands on that binade's first value.
    r = np.rint(x / q) * q
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def _decoded(q8, k8, v8):
    return decode_e4m3(q8), decode_e4m3(k8), decode_e4m3(v8)


def forward(q8, k8, v8, dq, dk, dv, scale, causal):
    """Exact attention of the dequantised inputs: returns (O, LSE), float64.

    q8: [nq, d] uint8 e4m3 codes; k8, v8: [nk, d]; dq, dk, dv: descales.
    Rows sit at absolute positions nk - nq .. nk - 1 (nq = nk: square).
    """
    q, k, v = _decoded(q8, k8, v8)
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nk - nq, nk)
    s = scores(q * float(dq), k * float(dk), scale, causal, rows=rows)
    p, _, _, lse = softmax_rows(s)
    return (p @ v) * float(dv), lse


def forward_quantised_p(q8, k8, v8, dq, dk, dv, scale, causal, p_scale=256.0):
    """Attention with the probabilities rounded to e4m3 before the product with V.

    Returns (O, LSE, aux) where aux holds the float32 exponent arguments
    x = S - m (natural-log units, [nq, nk]) and the rounded Pq, for the tests'
    error bounds.  Fully masked rows give O = 0 and LSE = -inf.
    """
    q, k, v = _decoded(q8, k8, v8)
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nk - nq, nk)
    s = scores(q * float(dq), k * float(dk), scale, causal, rows=rows)
    m = np.max(s, axis=1, keepdims=True) if nk else np.full((nq, 1), -np.inf)
    live = np.isfinite(m[:, 0])
    s32 = s.astype(np.float32)
    m32 = np.where(np.isfinite(m), m, 0.0).astype(np.float32)
    x = (s32 - m32).astype(np.float32)                      # -inf where masked
    p = np.exp(x).astype(np.float32)                        # float32 decision
    pq = round_e4m3(np.float64(p_scale) * p.astype(np.float64))
    l = p.astype(np.float64).sum(axis=1)
    denom = np.where(live, p_scale * l, 1.0)
    o = (pq @ v) * float(dv) / denom[:, None]
    o[~live] = 0.0
    lse = np.where(live, m[:, 0] + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse, {"x": x, "p": p, "pq": pq, "l": l}


def forward_quantised_p_online(q8, k8, v8, dq, dk, dv, scale, causal, block=64, p_scale=256.0):
    """forward_quantised_p with p rounded against the running maximum of the
    online softmax over blocks of `block` keys (see the module notes).

    Returns (O, LSE, aux); aux["x"] holds, per (row, key), the float32
    exponent argument S - m_b the key's p was formed from (-inf where masked),
    aux["p"] that p, aux["pq"] its rounded 2^8 p (before any rescale),
    aux["mref"] the maximum m_b it was taken against (-inf before the row's
    first visible key), aux["m"] the final maximum and aux["l"] the final
    running sum of p (relative to the final maximum).
    """
    q, k, v = _decoded(q8, k8, v8)
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nk - nq, nk)
    s = scores(q * float(dq), k * float(dk), scale, causal, rows=rows)
    s32 = s.astype(np.float32)
    m = np.full(nq, -np.inf)              # running maximum (float64 of float32 scores)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    xs = np.full((nq, nk), -np.inf, dtype=np.float32)
    ps = np.zeros((nq, nk), dtype=np.float32)
    pqs = np.zeros((nq, nk))
    mref = np.full((nq, nk), -np.inf)
    for j0 in range(0, nk, block):
        sb = s32[:, j0:j0 + block]
        m_new = np.maximum(m, sb.max(axis=1).astype(np.float64)) if sb.shape[1] else m
        grow = np.isfinite(m_new)
        alpha = np.where(grow & np.isfinite(m), np.exp(np.where(grow, m - m_new, 0.0)), 0.0)
        acc *= alpha[:, None]
        l *= alpha
        m = m_new
        m32 = np.where(grow, m, 0.0).astype(np.float32)[:, None]
        x = (sb - m32).astype(np.float32)
        p = np.exp(x).astype(np.float32)
        pq = round_e4m3(np.float64(p_scale) * p.astype(np.float64))
        acc += pq @ v[j0:j0 + block]
        l += p.astype(np.float64).sum(axis=1)
        xs[:, j0:j0 + block], ps[:, j0:j0 + block], pqs[:, j0:j0 + block] = x, p, pq
        mref[:, j0:j0 + block] = m[:, None]
    live = np.isfinite(m)
    denom = np.where(live, p_scale * l, 1.0)
    o = acc * float(dv) / denom[:, None]
    o[~live] = 0.0
    lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse, {"x": xs, "p": ps, "pq": pqs, "mref": mref, "m": m, "l": l}


def truncate_bits(x, bits):
    """x rounded toward zero to `bits` significant bits (float64 in and out)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.trunc(m * 2.0 ** bits) / 2.0 ** bits, e)


def _narrow_dot_blocks(a, b, acc_bits, kblk=64):
    """a @ b with the inner dimension taken in blocks of `kblk`: inside a block
    the products are added one by one to a sum truncated to `acc_bits` bits
    after each addition; each block's sum is then added to a float32 total."""
    n = a.shape[1]
    total = np.zeros((a.shape[0], b.shape[1]), dtype=np.float32)
    for c0 in range(0, n, kblk):
        part = np.zeros((a.shape[0], b.shape[1]))
        for c in range(c0, min(c0 + kblk, n)):
            part = truncate_bits(part + a[:, c:c + 1] * b[c:c + 1, :], acc_bits)
        total = (total + part.astype(np.float32)).astype(np.float32)
    return total.astype(np.float64)


def forward_narrow_accumulator(q8, k8, v8, dq, dk, dv, scale, causal, acc_bits=16, block=64,
                               p_scale=256.0):
    """The rounded-P online forward with both products summed through a narrow
    accumulator of `acc_bits` bits (see the module notes): returns (O, LSE).

    Scores: the code values of Q and K (products of two e4m3 values are exact)
    summed per 64 of d, then multiplied by scale * dq * dk in float32.  P V:
    the e4m3 values of 2^8 p against the running maximum of each block of
    `block` keys, times the code values of V, summed per 64 keys.
    """
    q, k, v = _decoded(q8, k8, v8)
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nk - nq, nk)
    raw = _narrow_dot_blocks(q, k.T, acc_bits)
    s32 = (raw.astype(np.float32) * np.float32(float(scale) * float(dq) * float(dk))).astype(np.float32)
    if causal:
        s32 = np.where(np.arange(nk)[None, :] > rows[:, None], np.float32(-np.inf), s32)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    for j0 in range(0, nk, block):
        sb = s32[:, j0:j0 + block]
        m_new = np.maximum(m, sb.max(axis=1).astype(np.float64))
        grow = np.isfinite(m_new)
        alpha = np.where(grow & np.isfinite(m), np.exp(np.where(grow, m - m_new, 0.0)), 0.0)
        acc *= alpha[:, None]
        l *= alpha
        m = m_new
        m32 = np.where(grow, m, 0.0).astype(np.float32)[:, None]
        p = np.exp((sb - m32).astype(np.float32)).astype(np.float32)
        pq = round_e4m3(np.float64(p_scale) * p.astype(np.float64))
        acc += _narrow_dot_blocks(pq, v[j0:j0 + block], acc_bits)
        l += p.astype(np.float64).sum(axis=1)
    live = np.isfinite(m)
    denom = np.where(live, p_scale * l, 1.0)
    o = acc * float(dv) / denom[:, None]
    o[~live] = 0.0
    lse = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse
