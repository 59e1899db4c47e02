"""Checks that pin the dropout oracle (oracle/dropout.py) to facts other than itself.

  * Philox4x32-10 reproduces the known-answer vectors published with the
    generator's reference implementation (Random123): counter and key all
    zero, all ones, and the digits of pi.
  * The mask keeps a fraction 1 - p of the elements (within 5 sigma of the
    binomial spread) for several p; p = 0 keeps everything; different seeds,
    offsets and heads give different masks; element (i, j) is 16-bit field
    4 (j div 8 mod 2) + j mod 4 of the call on counter word
    2 (j div 16) + (j div 4 mod 2), computed here from single calls written
    out per element; every field of a call serves exactly one key; the
    threshold rounds p 2^16 to the nearest integer and the kept scale is
    2^16 / (2^16 - threshold), checked on hand values.
  * p = 0 reduces forward and backward to plain attention (oracle.attention).
  * With the mask fixed, dQ, dK, dV agree with central finite differences of
    sum(O * dO), causal and not; sum_j dK_j = 0 and D = rowsum(dO * O) still
    hold (dropout leaves the softmax rows alone).
  * Averaged over many masks the output approaches plain attention (the
    1 / (1 - p) scaling makes dropout unbiased), within 5 standard errors.
"""
from __future__ import annotations

import numpy as np

import oracle.attention as att

KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def pin_philox_kat(drop):
    for ctr, key, expect in KAT:
        got = drop.philox4x32_10(np.array(ctr, dtype=np.uint64), key)
        assert [int(x) for x in got] == list(expect), f"Philox({ctr}, {key}) = {[hex(int(x)) for x in got]}"


def pin_mask(drop):
    rows = np.arange(300)
    for p in (0.1, 0.25, 0.5, 0.9):
        keep = drop.keep_mask(3, rows, 1000, p, seed=0x1234567890AB, offset=5)
        n = keep.size
        frac = keep.mean()
        sigma = np.sqrt(p * (1 - p) / n)
        assert abs(frac - (1 - p)) <= 5 * sigma, f"p = {p}: kept {frac:.4f}"
    assert drop.keep_mask(0, rows, 64, 0.0, seed=7).all(), "p = 0 drops something"
    base = drop.keep_mask(1, rows, 256, 0.5, seed=11, offset=0)
    for other in (drop.keep_mask(1, rows, 256, 0.5, seed=12, offset=0),
                  drop.keep_mask(1, rows, 256, 0.5, seed=11, offset=1),
                  drop.keep_mask(2, rows, 256, 0.5, seed=11, offset=0)):
        assert 0.4 < np.mean(other != base) < 0.6, "masks of different seeds/offsets/heads agree"
    # hand values of the threshold and the scale of kept probabilities
    assert drop.threshold(0.0) == 0 and drop.threshold(0.5) == 32768
    assert drop.threshold(0.1) == 6554            # 6553.6 rounds up
    assert drop.threshold(0.25) == 16384 and drop.threshold(1 - 2 ** -20) == 65535
    assert drop.keep_scale(0.5) == 2.0 and drop.keep_scale(0.75) == 4.0 and drop.keep_scale(0.0) == 1.0
    assert abs(drop.keep_scale(0.1) - 65536 / 58982) < 1e-15
    # element by element from single generator calls
    seed, bh, off, p = 0xDEADBEEFCAFE, 5, 9, 0.3
    keep = drop.keep_mask(bh, np.array([0, 7, 41]), 45, p, seed=seed, offset=off)
    thr = 19661                                    # round(0.3 * 65536) = round(19660.8)
    assert drop.threshold(p) == thr
    for a, i in enumerate((0, 7, 41)):
        for j in range(45):
            ctr0 = 2 * (j // 16) + (j // 4) % 2
            field = 4 * ((j // 8) % 2) + j % 4
            w = int(drop.philox4x32_10(np.array([ctr0, i, bh, off], dtype=np.uint64),
                                       (seed & 0xFFFFFFFF, seed >> 32))[field // 2])
            half = (w >> (16 * (field % 2))) & 0xFFFF
            assert keep[a, j] == (half >= thr), f"element ({i}, {j})"
    # one call serves keys 16a + 4b + {0..3, 8..11}: eight distinct fields
    c, f = drop.counter_field(np.arange(256))
    pairs = set(zip(c.tolist(), f.tolist()))
    assert len(pairs) == 256 and set(f.tolist()) == set(range(8)), "keys share a field"
    for a in range(16):
        for b in range(2):
            keys = [16 * a + 4 * b + e for e in (0, 1, 2, 3, 8, 9, 10, 11)]
            assert set(c[keys].tolist()) == {2 * a + b} and sorted(f[keys].tolist()) == list(range(8))


def _inputs(seed, n, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)) for _ in range(4))


def pin_p0_is_plain(drop):
    q, k, v, do = _inputs(1, 20, 8)
    keep = np.ones((20, 20), dtype=bool)
    for causal in (False, True):
        o, lse = drop.forward(q, k, v, 0.4, causal, keep, 0.0)
        o_r, lse_r = att.forward(q, k, v, 0.4, causal)
        _close(o, o_r, 1e-13, "p = 0 forward")
        _close(lse, lse_r, 1e-13, "p = 0 LSE")
        g = drop.backward(q, k, v, do, 0.4, causal, keep, 0.0)
        g_r = att.backward(q, k, v, do, 0.4, causal)
        for name, a, b in zip(("dQ", "dK", "dV"), g[:3], g_r[:3]):
            _close(a, b, 1e-12, f"p = 0 {name}")


def pin_finite_differences(drop):
    n, d, p, scale = 9, 4, 0.3, 0.7
    q, k, v, do = _inputs(2, n, d)
    keep = drop.keep_mask(0, np.arange(n), n, p, seed=99)
    assert 0 < keep.sum() < keep.size
    for causal in (False, True):
        dq, dk, dv, dvec = drop.backward(q, k, v, do, scale, causal, keep, p)
        grads = {"q": dq, "k": dk, "v": dv}
        for name in "qkv":
            x = {"q": q, "k": k, "v": v}
            num = np.zeros_like(x[name])
            for idx in np.ndindex(*num.shape):
                for sgn in (1, -1):
                    xx = {t: a.copy() for t, a in x.items()}
                    xx[name][idx] += sgn * 1e-6
                    o, _ = drop.forward(xx["q"], xx["k"], xx["v"], scale, causal, keep, p)
                    num[idx] += sgn * (o * do).sum() / 2e-6
            _close(grads[name], num, 1e-6, f"d{name.upper()} vs finite differences (causal={causal})")
        assert np.abs(dk.sum(axis=0)).max() < 1e-12, "sum_j dK_j != 0"
        o, _ = drop.forward(q, k, v, scale, causal, keep, p)
        _close(dvec, (o * do).sum(axis=1), 1e-12, "D = rowsum(dO * O)")


def pin_unbiased(drop):
    n, d, p = 6, 4, 0.5
    q, k, v, _ = _inputs(3, n, d)
    outs = np.stack([drop.forward(q, k, v, 0.5, True, drop.keep_mask(0, np.arange(n), n, p, seed=s), p)[0]
                     for s in range(2000)])
    ref, _ = att.forward(q, k, v, 0.5, True)
    se = outs.std(axis=0) / np.sqrt(outs.shape[0])
    assert (np.abs(outs.mean(axis=0) - ref) <= 5 * se + 1e-12).all(), "dropout output is biased"


DROPOUT_PINS = [pin_philox_kat, pin_mask, pin_p0_is_plain, pin_finite_differences, pin_unbiased]
