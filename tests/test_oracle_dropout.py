"""The dropout oracle against its pins, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle.dropout as drop
from dropout_pins import DROPOUT_PINS


@pytest.mark.parametrize("pin", DROPOUT_PINS, ids=lambda p: p.__name__)
def test_dropout_oracle_pin(pin):
    pin(drop)


_orig = {n: getattr(drop, n) for n in ("philox4x32_10", "keep_mask", "forward", "backward", "threshold",
                                      "keep_scale", "counter_field")}


def _philox_wrong_multiplier(ctr, key):
    x = [np.asarray(ctr, dtype=np.uint64)[..., i] for i in range(4)]
    k0, k1 = int(key[0]), int(key[1])
    for _ in range(10):
        p0 = np.uint64(0xD2511F55) * x[0]
        p1 = np.uint64(0xCD9E8D57) * x[2]
        x = [(p1 >> np.uint64(32)) ^ x[1] ^ np.uint64(k0), p1 & np.uint64(0xFFFFFFFF),
             (p0 >> np.uint64(32)) ^ x[3] ^ np.uint64(k1), p0 & np.uint64(0xFFFFFFFF)]
        k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return np.stack(x, axis=-1).astype(np.uint32)


def _mask_rows_keys_swapped(bh, rows, nk, p, seed, offset=0):
    rows = np.asarray(rows)
    full = _orig["keep_mask"](bh, np.arange(max(nk, rows.max() + 1)), max(nk, rows.max() + 1), p, seed, offset)
    return full.T[rows][:, :nk]


def _mask_inverted(bh, rows, nk, p, seed, offset=0):
    return ~_orig["keep_mask"](bh, rows, nk, p, seed, offset) if p > 0 else _orig["keep_mask"](bh, rows, nk, p, seed, offset)


def _mask_halves_swapped(bh, rows, nk, p, seed, offset=0):
    """Reads the high 16 bits where the low ones are meant and vice versa."""
    rows = np.asarray(rows, dtype=np.uint64)
    c, f = drop.counter_field(np.arange(nk))
    ctr = np.zeros((rows.size, nk, 4), dtype=np.uint64)
    ctr[..., 0], ctr[..., 1], ctr[..., 2], ctr[..., 3] = c[None, :], rows[:, None], bh, offset
    words = drop.philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, int(seed) >> 32)).astype(np.uint64)
    word = np.take_along_axis(words, (f >> np.uint64(1)).astype(np.int64)[None, :, None].repeat(rows.size, 0), 2)[..., 0]
    field = (word >> (np.uint64(16) * (np.uint64(1) - (f & np.uint64(1))))[None, :]) & np.uint64(0xFFFF)
    return field >= np.uint64(drop.threshold(p))


def _counter_field_per_4_keys(j):
    """The old one-word-per-element layout: counter j div 4, field 2 (j mod 4)."""
    j = np.asarray(j, dtype=np.uint64)
    return j >> np.uint64(2), (j & np.uint64(3)) << np.uint64(1)


def _threshold_floor(p):
    return min(int(np.floor(float(p) * 65536.0)), 65535)


def _scale_one_over_1_minus_p(p):
    return 1.0 / (1.0 - float(p))


def _forward_variant(kind):
    def forward(q, k, v, scale, causal, keep, p):
        pm, _, _, lse = drop.softmax_rows(drop.scores(q, k, scale, causal))
        if kind == "no_rescale":
            z = np.where(keep, 1.0, 0.0)
        else:
            z = np.where(keep, drop.keep_scale(p), 0.0)
        pz = pm * z
        if kind == "renormalised":
            pz = pz / np.maximum(pz.sum(axis=1, keepdims=True), 1e-300)
        return pz @ np.asarray(v, dtype=np.float64), lse
    return forward


def _backward_variant(kind):
    def backward(q, k, v, do, scale, causal, keep, p):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        pm, _, _, _ = drop.softmax_rows(drop.scores(q, k, scale, causal))
        z = np.where(keep, drop.keep_scale(p), 0.0)
        dv = (pm * (1.0 if kind == "dv_unmasked" else z)).T @ do
        dp = (do @ v.T) * (1.0 if kind == "dp_unmasked" else z)
        dvec = (pm * dp).sum(axis=1)
        ds = pm * (dp - dvec[:, None])
        return scale * ds @ k, scale * ds.T @ q, dv, dvec
    return backward


MUTANTS = {
    "philox_wrong_multiplier": ("philox4x32_10", _philox_wrong_multiplier),
    "mask_rows_and_keys_swapped": ("keep_mask", _mask_rows_keys_swapped),
    "mask_keeps_the_dropped": ("keep_mask", _mask_inverted),
    "mask_16_bit_halves_swapped": ("keep_mask", _mask_halves_swapped),
    "counter_and_field_of_the_old_layout": ("counter_field", _counter_field_per_4_keys),
    "threshold_rounded_down": ("threshold", _threshold_floor),
    "scale_not_from_the_threshold": ("keep_scale", _scale_one_over_1_minus_p),
    "forward_without_1_over_keep": ("forward", _forward_variant("no_rescale")),
    "forward_renormalised_after_dropout": ("forward", _forward_variant("renormalised")),
    "backward_dP_unmasked": ("backward", _backward_variant("dp_unmasked")),
    "backward_dV_unmasked": ("backward", _backward_variant("dv_unmasked")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_dropout_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(drop, attr, fn)
    caught = []
    for pin in DROPOUT_PINS:
        try:
            pin(drop)
        except Exception as e:  # a failed check or an error both expose the mistake
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"no pin caught the planted mistake {name}"


def test_dropout_unmutated_templates_pass(monkeypatch):
    monkeypatch.setattr(drop, "forward", _forward_variant("none"))
    monkeypatch.setattr(drop, "backward", _backward_variant("none"))
    for pin in DROPOUT_PINS:
        pin(drop)
