"""Checks that pin the FP8 CPU oracle (oracle/fp8.py) to facts other than itself.

Each pin takes the oracle module (or a copy with a planted mistake) and raises
AssertionError when it disagrees with a library routine, a closed form or a
bound that follows from the format:

  * decode_e4m3 of every code agrees with torch's float8_e4m3fn dtype (the OCP
    E4M3 format), and with hand values: 0x38 = 1, 0x7E = 448, 0x08 = 2^-6,
    0x01 = 2^-9, 0xB8 = -1, 0x7F and 0xFF are NaN.
  * round_e4m3 agrees with torch's float32 -> float8_e4m3fn conversion (round
    to nearest, ties to even) on random values and on every exact midpoint
    between adjacent codes, and leaves every code's value unchanged.
  * Q = 0 makes every score equal: O is dv times the mean of the decoded V rows
    and LSE = ln(number of keys).
  * The descales act as scalars: forward(dq, dk, dv) equals the fp64 attention
    of the decoded values multiplied by their descales.
  * Probabilities that are powers of two stay exact after the factor 2^8 and
    rounding, so forward_quantised_p equals forward.
  * A two-key example with scores (2c, c), c = -ln 0.3, so p = (1, 0.3):
    2^8 * 0.3 = 76.8 rounds to 80, O = dv (256 v0 + 80 v1) / (256 * 1.3) and
    LSE = 2c + ln 1.3.
  * The online variant equals the final-maximum one when one block holds all
    keys, and on rows whose maximum lies in the first block.
  * A three-key online example, blocks of two: scores (0, -c, c), c = -ln 0.3.
    Block one rounds 2^8 (1, 0.3) to (256, 80) against the maximum 0; block
    two raises the maximum to c and rescales by e^-c = 0.3, so
    O = dv (0.3 (256 v_a + 80 v_b) + 256 v_c) / (256 (0.3 (1 + 0.3) + 1)),
    where rounding against the final maximum would give (80, 24, 256).
  * On random inputs the rounded-P results (both variants) lie within the bound
    dv sum_j max(2^-4 y_ij, 2^-10) |V_j| / (256 l_i), y = 256 p, of the exact
    one, and the bound is not met trivially (the two differ).
  * truncate_bits keeps the leading bits of the binary expansion: 1.9999 to 2
    bits is 1.5, -5.5 to 2 bits is -4, 3 to 2 bits stays 3, and to 24 bits it
    agrees with numpy's float32 conversion wherever that rounds down in
    magnitude.
  * The narrow-accumulator model with a 53-bit accumulator is the online
    rounded-P result (up to the float32 totals); with integer-coded Q and K of
    magnitude <= 15 and a 15-bit accumulator every score is an exact integer
    sum, so it equals the 53-bit model; with an 8-bit accumulator on spread
    inputs it differs.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def _codes(x):
    """e4m3 codes (uint8) of float values, by torch's conversion."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_decode(fp8):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = fp8.decode_e4m3(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"decode differs from torch float8_e4m3fn at codes {np.nonzero(~same)[0][:8]}"
    hand = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0xB8: -1.0, 0x00: 0.0}
    for c, v in hand.items():
        assert fp8.decode_e4m3(np.array([c], np.uint8))[0] == v, f"code {c:#x}"
    assert np.isnan(fp8.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def pin_round(fp8):
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 60, rng.random(20000) * 2.0 ** -5,
                        -rng.random(2000) * 448])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    got = fp8.round_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref), f"round differs from torch on {np.sum(got != ref)} values"
    vals = np.sort(np.unique(fp8.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in float32
    ref = torch.from_numpy(np.concatenate([mids, -mids])).to(torch.float8_e4m3fn).double().numpy()
    got = fp8.round_e4m3(np.concatenate([mids, -mids]).astype(np.float64))
    assert np.array_equal(got, ref), "ties are not rounded to the even code"
    assert np.array_equal(fp8.round_e4m3(vals), vals), "rounding moves an e4m3 value"
    hand = [(76.8, 80.0), (1 + 1 / 16, 1.0), (1 + 3 / 16, 1.25), (248.0, 256.0),
            (2.0 ** -10, 0.0), (3 * 2.0 ** -10, 2.0 ** -8)]
    for a, b in hand:
        assert fp8.round_e4m3(np.array([a]))[0] == b, f"round({a}) != {b}"


def pin_zero_query(fp8):
    rng = np.random.default_rng(3)
    nk, d = 37, 16
    q8 = _codes(np.zeros((5, d)))
    k8 = _codes(rng.standard_normal((nk, d)))
    v8 = _codes(rng.standard_normal((nk, d)))
    dv = 0.75
    o, lse = fp8.forward(q8, k8, v8, 2.0, 0.5, dv, 0.3, False)
    mean_v = fp8.decode_e4m3(v8).mean(axis=0) * dv
    _close(o, np.broadcast_to(mean_v, o.shape), 1e-13, "Q = 0: O is the mean of V")
    _close(lse, np.full(5, math.log(nk)), 1e-13, "Q = 0: LSE = ln nk")


def pin_descales(fp8):
    rng = np.random.default_rng(4)
    nq, nk, d = 9, 23, 32
    q8, k8, v8 = (_codes(rng.standard_normal((n, d)) * 2) for n in (nq, nk, nk))
    dq, dk, dv, scale = 0.37, 1.9, 0.61, d ** -0.5
    for causal in (False, True):
        o, lse = fp8.forward(q8, k8, v8, dq, dk, dv, scale, causal)
        q = torch.from_numpy(q8.copy()).view(torch.float8_e4m3fn).double() * dq
        k = torch.from_numpy(k8.copy()).view(torch.float8_e4m3fn).double() * dk
        v = torch.from_numpy(v8.copy()).view(torch.float8_e4m3fn).double() * dv
        s = scale * q @ k.T
        if causal:   # rows are the last nq positions of nk
            hidden = torch.arange(nk)[None, :] > torch.arange(nk - nq, nk)[:, None]
            s = s.masked_fill(hidden, -math.inf)
        ref_o = torch.softmax(s, dim=1) @ v
        _close(o, ref_o.numpy(), 1e-12, f"descaled forward (causal={causal})")
        _close(lse, torch.logsumexp(s, dim=1).numpy(), 1e-12, f"descaled LSE (causal={causal})")


def pin_exact_powers_of_two(fp8):
    # Scores -j ln 2 give p_j = 2^-j; 2^8 p_j = 2^(8-j) are e4m3 values.
    d = 16
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((8, d)); k[:, 0] = -np.arange(8)
    rng = np.random.default_rng(5)
    v8 = _codes(rng.standard_normal((8, d)))
    scale = math.log(2.0)
    o_q, lse_q, aux = fp8.forward_quantised_p(_codes(q), _codes(k), v8, 1.0, 1.0, 1.25, scale, False)
    o, lse = fp8.forward(_codes(q), _codes(k), v8, 1.0, 1.0, 1.25, scale, False)
    assert np.array_equal(aux["pq"][0], 2.0 ** (8 - np.arange(8))), "2^8 p is not 2^(8-j)"
    _close(o_q, o, 1e-6, "representable probabilities: rounded-P forward equals forward")
    _close(lse_q, lse, 1e-6, "representable probabilities: LSE")


def pin_worked_two_keys(fp8):
    # scale c = -ln 0.3 > 0, q = e0, keys 2 e0 and e0: s = (2c, c), the row
    # maximum is 2c, p = (1, 0.3), and 2^8 * 0.3 = 76.8 rounds to 80.
    d = 8
    c = -math.log(0.3)
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((2, d)); k[0, 0] = 2.0; k[1, 0] = 1.0
    v = np.zeros((2, d)); v[0, :] = 1.0; v[1, :] = -2.0
    dv = 0.5
    o, lse, aux = fp8.forward_quantised_p(_codes(q), _codes(k), _codes(v), 1.0, 1.0, dv, c, False)
    assert np.array_equal(aux["pq"][0], [256.0, 80.0]), f"Pq = {aux['pq'][0]}"
    expect = dv * (256 * 1.0 + 80 * -2.0) / (256 * 1.3)
    _close(o, np.full((1, d), expect), 1e-6, "two-key worked example")
    _close(lse, [2 * c + math.log(1.3)], 1e-6, "two-key LSE")


def _bound(fp8, p_exact, v8, dv):
    """Worst-case |O_rounded - O_exact| per element from the e4m3 rounding of 256 p."""
    y = 256.0 * p_exact
    err = np.maximum(2.0 ** -4 * y, 2.0 ** -10)
    err = np.where(p_exact > 0, err, 0.0)
    l = p_exact.sum(axis=1)
    return dv * (err @ np.abs(fp8.decode_e4m3(v8))) / (256.0 * l[:, None])


def pin_rounding_bound(fp8):
    rng = np.random.default_rng(6)
    nq = nk = 48
    d = 32
    q8, k8, v8 = (_codes(rng.standard_normal((n, d))) for n in (nq, nk, nk))
    for causal in (False, True):
        o, lse = fp8.forward(q8, k8, v8, 1.1, 0.9, 0.7, d ** -0.5, causal)
        o_q, lse_q, _ = fp8.forward_quantised_p(q8, k8, v8, 1.1, 0.9, 0.7, d ** -0.5, causal)
        o_o, lse_o, _ = fp8.forward_quantised_p_online(q8, k8, v8, 1.1, 0.9, 0.7, d ** -0.5, causal, block=8)
        q = fp8.decode_e4m3(q8) * 1.1
        k = fp8.decode_e4m3(k8) * 0.9
        s = d ** -0.5 * q @ k.T
        if causal:
            s = np.where(np.arange(nk)[None, :] > np.arange(nq)[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        bound = _bound(fp8, p, v8, 0.7) + 1e-6
        for name, oo, ll in (("final maximum", o_q, lse_q), ("online", o_o, lse_o)):
            diff = np.abs(oo - o)
            assert (diff <= bound).all(), f"{name}: rounded-P result outside the rounding bound (causal={causal})"
            assert diff.max() > 1e-4, f"{name}: rounding P to e4m3 changed nothing"
            _close(ll, lse, 1e-5, f"{name}: LSE does not depend on the rounding (causal={causal})")


def pin_online_matches_final_max(fp8):
    rng = np.random.default_rng(8)
    nq = nk = 40
    d = 16
    q8, k8, v8 = (_codes(rng.standard_normal((n, d))) for n in (nq, nk, nk))
    for causal in (False, True):
        ref = fp8.forward_quantised_p(q8, k8, v8, 1.0, 1.0, 0.5, d ** -0.5, causal)
        got = fp8.forward_quantised_p_online(q8, k8, v8, 1.0, 1.0, 0.5, d ** -0.5, causal, block=64)
        _close(got[0], ref[0], 1e-12, f"online, one block: O (causal={causal})")
        _close(got[1], ref[1], 1e-12, f"online, one block: LSE (causal={causal})")
    # a sink key 0 holds every row's maximum: blocks of 8 round as the final maximum does
    k = rng.standard_normal((nk, d)); k[:, 0] = 0.0; k[0, 0] = 12.0
    q = rng.standard_normal((nq, d)); q[:, 0] = 4.0
    q8, k8 = _codes(q), _codes(k)
    ref = fp8.forward_quantised_p(q8, k8, v8, 1.0, 1.0, 0.5, d ** -0.5, True)
    got = fp8.forward_quantised_p_online(q8, k8, v8, 1.0, 1.0, 0.5, d ** -0.5, True, block=8)
    _close(got[0], ref[0], 1e-12, "online, maximum in the first block: O")


def pin_online_worked_three_keys(fp8):
    d = 8
    c = -math.log(0.3)
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((3, d)); k[1, 0] = -1.0; k[2, 0] = 1.0
    v = np.zeros((3, d)); v[0, :] = 1.0; v[1, :] = -2.0; v[2, :] = 0.5
    dv = 0.75
    o, lse, aux = fp8.forward_quantised_p_online(_codes(q), _codes(k), _codes(v), 1.0, 1.0, dv, c,
                                                 False, block=2)
    assert np.array_equal(aux["pq"][0], [256.0, 80.0, 256.0]), f"online Pq = {aux['pq'][0]}"
    num = 0.3 * (256 * 1.0 + 80 * -2.0) + 256 * 0.5
    den = 256 * (0.3 * (1 + 0.3) + 1)
    _close(o, np.full((1, d), dv * num / den), 1e-6, "three-key online example")
    _close(lse, [c + math.log(0.3 * 1.3 + 1)], 1e-6, "three-key online LSE")
    _, _, aux_f = fp8.forward_quantised_p(_codes(q), _codes(k), _codes(v), 1.0, 1.0, dv, c, False)
    assert np.array_equal(aux_f["pq"][0], [80.0, 24.0, 256.0]), f"final-maximum Pq = {aux_f['pq'][0]}"


def pin_truncate_bits(fp8):
    got = fp8.truncate_bits(np.array([1.9999, -5.5, 3.0, 0.0, 1.0]), 2)
    assert np.array_equal(got, [1.5, -4.0, 3.0, 0.0, 1.0]), f"truncate_bits to 2 bits: {got}"
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000) * np.exp2(rng.integers(-20, 20, 10000))
    f = x.astype(np.float32).astype(np.float64)
    down = np.abs(f) <= np.abs(x)
    assert np.array_equal(fp8.truncate_bits(x, 24)[down], f[down]), "truncate_bits(24) vs float32"
    assert (np.abs(fp8.truncate_bits(x, 24)) <= np.abs(x)).all(), "truncation must not grow |x|"


def pin_narrow_accumulator(fp8):
    rng = np.random.default_rng(23)
    nq, nk, d = 40, 150, 128
    q = _codes(rng.standard_normal((nq, d)).astype(np.float32) * 4)
    k = _codes(rng.standard_normal((nk, d)).astype(np.float32) * 4)
    v = _codes(rng.standard_normal((nk, d)).astype(np.float32))
    sc = 0.01
    for causal in (False, True):
        o53, lse53 = fp8.forward_narrow_accumulator(q, k, v, 1.0, 1.0, 1.0, sc, causal, acc_bits=53)
        o_on, lse_on, _ = fp8.forward_quantised_p_online(q, k, v, 1.0, 1.0, 1.0, sc, causal, block=64)
        _close(o53, o_on, 2e-4, "53-bit accumulator = online rounded-P O")
        _close(lse53, lse_on, 1e-5, "53-bit accumulator = online rounded-P LSE")
        o8, _ = fp8.forward_narrow_accumulator(q, k, v, 1.0, 1.0, 1.0, sc, causal, acc_bits=8)
        assert np.abs(o8 - o53).max() > 1e-3, "an 8-bit accumulator should change O"
    qi = _codes(np.clip(np.rint(rng.standard_normal((nq, d)) * 4), -15, 15).astype(np.float32))
    ki = _codes(np.clip(np.rint(rng.standard_normal((nk, d)) * 4), -15, 15).astype(np.float32))
    for causal in (False, True):
        o15, lse15 = fp8.forward_narrow_accumulator(qi, ki, v, 0.25, 0.25, 1.0, sc, causal, acc_bits=15)
        o53, lse53 = fp8.forward_narrow_accumulator(qi, ki, v, 0.25, 0.25, 1.0, sc, causal, acc_bits=53)
        # scores exact either way; the P V sums may differ by the 15-bit rounding
        _close(lse15, lse53, 0.0, "integer scores with a 15-bit accumulator")
        _close(o15, o53, 2e-3, "integer scores with a 15-bit accumulator, O")


FP8_PINS = [
    pin_decode, pin_round, pin_zero_query, pin_descales, pin_exact_powers_of_two,
    pin_worked_two_keys, pin_online_matches_final_max, pin_online_worked_three_keys,
    pin_rounding_bound, pin_truncate_bits, pin_narrow_accumulator,
]
