"""The FP8 oracle against its pins, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle.fp8 as fp8
from fp8_pins import FP8_PINS


@pytest.mark.parametrize("pin", FP8_PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_pin(pin):
    pin(fp8)


_orig = {n: getattr(fp8, n) for n in ("decode_e4m3", "round_e4m3", "forward", "forward_quantised_p",
                                      "forward_quantised_p_online")}


def _decode_bias8(codes):
    # the e4m3 "fnuz" variant: exponent bias 8, so every value is halved
    return _orig["decode_e4m3"](codes) / 2.0


def _round_toward_zero(x):
    x = np.asarray(x, dtype=np.float64)
    q = fp8.e4m3_spacing(x)
    return np.clip(np.trunc(x / q) * q, -fp8.E4M3_MAX, fp8.E4M3_MAX)


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    q = fp8.e4m3_spacing(x)
    return np.clip(np.sign(x) * np.floor(np.abs(x) / q + 0.5) * q, -fp8.E4M3_MAX, fp8.E4M3_MAX)


def _forward_dv_in_scores(q8, k8, v8, dq, dk, dv, scale, causal):
    return _orig["forward"](q8, k8, v8, dq * dv, dk, 1.0, scale, causal)


def _qp_variant(kind):
    def forward_quantised_p(q8, k8, v8, dq, dk, dv, scale, causal, p_scale=256.0):
        o, lse, aux = _orig["forward_quantised_p"](q8, k8, v8, dq, dk, dv, scale, causal, p_scale)
        v = fp8.decode_e4m3(v8)
        pq, l = aux["pq"], aux["l"]
        if kind == "normalise_by_rounded":
            o = (pq @ v) * dv / pq.sum(axis=1, keepdims=True)
        elif kind == "no_p_scale":
            o = (pq @ v) * dv / l[:, None]
        elif kind == "unrounded":
            o = (aux["p"].astype(np.float64) @ v) * dv / l[:, None]
        elif kind == "max_too_low":
            # p rounded against m - 1 instead of the row maximum m
            p = np.exp(aux["x"].astype(np.float64) + 1.0)
            pq = fp8.round_e4m3(p_scale * p)
            o = (pq @ v) * dv / (p_scale * p.sum(axis=1, keepdims=True))
        return o, lse, {**aux, "pq": pq}
    return forward_quantised_p


def _online_variant(kind):
    def forward_quantised_p_online(q8, k8, v8, dq, dk, dv, scale, causal, block=64, p_scale=256.0):
        if kind == "final_maximum":
            return _orig["forward_quantised_p"](q8, k8, v8, dq, dk, dv, scale, causal, p_scale)
        q, k, v = (fp8.decode_e4m3(x) for x in (q8, k8, v8))
        nq, nk = q.shape[0], k.shape[0]
        s = fp8.scores(q * dq, k * dk, scale, causal, rows=np.arange(nk - nq, nk)).astype(np.float32)
        m = np.full(nq, -np.inf); l = np.zeros(nq); acc = np.zeros((nq, v.shape[1]))
        pqs = np.zeros((nq, nk))
        for j0 in range(0, nk, block):
            sb = s[:, j0:j0 + block]
            m_new = np.maximum(m, sb.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            if kind != "no_rescale":
                acc *= alpha[:, None]
            l *= alpha
            m = m_new
            p = np.exp((sb - m[:, None].astype(np.float32)).astype(np.float32))
            pq = fp8.round_e4m3(p_scale * p.astype(np.float64))
            acc += pq @ v[j0:j0 + block]
            l += p.astype(np.float64).sum(axis=1)
            pqs[:, j0:j0 + block] = pq
        return acc * dv / (p_scale * l[:, None]), m + np.log(l), {"pq": pqs, "l": l}
    return forward_quantised_p_online


MUTANTS = {
    "decode_bias_8": ("decode_e4m3", _decode_bias8),
    "round_toward_zero": ("round_e4m3", _round_toward_zero),
    "round_ties_away": ("round_e4m3", _round_ties_away),
    "forward_dv_in_scores": ("forward", _forward_dv_in_scores),
    "qp_normalised_by_rounded_p": ("forward_quantised_p", _qp_variant("normalise_by_rounded")),
    "qp_without_p_scale": ("forward_quantised_p", _qp_variant("no_p_scale")),
    "qp_not_rounded": ("forward_quantised_p", _qp_variant("unrounded")),
    "qp_wrong_row_maximum": ("forward_quantised_p", _qp_variant("max_too_low")),
    "online_without_rescale": ("forward_quantised_p_online", _online_variant("no_rescale")),
    "online_rounds_against_final_maximum": ("forward_quantised_p_online", _online_variant("final_maximum")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fp8, attr, fn)
    caught = []
    for pin in FP8_PINS:
        try:
            pin(fp8)
        except Exception as e:  # a failed check or an error both expose the mistake
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"no pin caught the planted mistake {name}"


def test_fp8_unmutated_template_passes(monkeypatch):
    monkeypatch.setattr(fp8, "forward_quantised_p", _qp_variant("none"))
    for pin in FP8_PINS:
        pin(fp8)


def test_fp8_unmutated_online_template_passes(monkeypatch):
    monkeypatch.setattr(fp8, "forward_quantised_p_online", _online_variant("none"))
    for pin in FP8_PINS:
        pin(fp8)


# The FP8 GPU parity bound (tests/fp8_bounds.py) rests on an assumed minimum
# accumulator width of the FP8 matrix instruction.  A model of a kernel with
# exactly that width (truncating after every addition) must stay inside the
# bound, and a model with a much narrower accumulator must not, so that the
# bound is shown to cover the assumption without being vacuous.
_ACC_CASES = [   # Nq, Nk, d, causal, integer-coded Q and K
    (256, 256, 64, True, True),
    (200, 333, 128, False, False),
    (300, 300, 128, True, False),
    (500, 200, 64, False, True),
    (1, 1, 64, False, True),
]


def _acc_ratios(acc_bits):
    import synth
    from fp8_bounds import loose_bound, lse_bound
    worst = 0.0
    for Nq, Nk, d, causal, qi in _ACC_CASES:
        host = synth.make_fp8_inputs(1, Nq, Nk, 1, d, seed=3000 + Nq + 7 * Nk + d, qk_int=qi)
        q8, k8, v8 = (host[x][0, :, 0] for x in "qkv")
        ds = host["descales"]
        sc = synth.f32(d ** -0.5)
        o_ex, lse_ex = fp8.forward(q8, k8, v8, *ds, sc, causal)
        o_m, lse_m = fp8.forward_narrow_accumulator(q8, k8, v8, *ds, sc, causal, acc_bits=acc_bits)
        r_o = float((np.abs(o_m - o_ex) / loose_bound(q8, k8, v8, ds, sc, causal, o_ex)).max())
        r_l = float((np.abs(lse_m - lse_ex) / lse_bound(q8, k8, ds, sc, causal, lse_ex)).max())
        worst = max(worst, r_o, r_l)
    return worst


def test_bound_covers_assumed_accumulator():
    from fp8_bounds import ACC_BITS
    assert _acc_ratios(ACC_BITS) <= 1.0


def test_bound_rejects_8_bit_accumulator():
    assert _acc_ratios(8) > 1.0
