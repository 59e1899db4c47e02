"""Plant plausible mistakes in the CPU oracle and check that some pin catches each.

Every mutant is a copy of one oracle function with one deliberate error (a
dropped term, a wrong sign or index, a transposed operand, a wrong mask).  The
oracle module is patched for the duration of one test only.
"""
import numpy as np
import pytest

import oracle.attention as ora
from oracle_pins import ALL_PINS


def _scores_noscale(q, k, scale, causal, rows=None):
    return _orig_scores(q, k, 1.0, causal, rows)


def _scores_transposed(q, k, scale, causal, rows=None):
    s = float(scale) * (np.asarray(k, float) @ np.asarray(q, float).T)
    if causal:
        s = np.where(np.arange(s.shape[1])[None, :] > np.arange(s.shape[0])[:, None], -np.inf, s)
    return s


def _mask_variant(cmp):
    def scores(q, k, scale, causal, rows=None):
        s = float(scale) * (np.asarray(q, float) @ np.asarray(k, float).T)
        if causal:
            qi = np.arange(s.shape[0]) if rows is None else np.asarray(rows)
            s = np.where(cmp(np.arange(s.shape[1])[None, :], qi[:, None]), -np.inf, s)
        return s
    return scores


def _softmax_no_log(s):
    p, m, l, lse = _orig_softmax(s)
    return p, m, l, m + l


def _softmax_columns(s):
    pt, m, l, lse = _orig_softmax(s.T)
    return pt.T, m, l, lse


def _forward_uses_k(q, k, v, scale, causal):
    p, _, _, lse = ora.softmax_rows(ora.scores(q, k, scale, causal))
    return p @ np.asarray(k, float), lse


def _backward_variant(kind):
    def backward(q, k, v, do, scale, causal, rows=None):
        q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
        p, _, _, _ = ora.softmax_rows(ora.scores(q, k, scale, causal, rows=rows))
        dv = p.T @ do if kind != "dv_untransposed" else p @ do
        dp = do @ v.T
        dvec = (p * dp).sum(axis=1)
        if kind == "drop_D":
            ds = p * dp
        elif kind == "flip_sign":
            ds = p * (dvec[:, None] - dp)
        else:
            ds = p * (dp - dvec[:, None])
        dq = (1.0 if kind == "dq_noscale" else scale) * (ds @ k)
        dk = scale * (ds.T @ q if kind != "dk_untransposed" else ds @ q)
        return dq, dk, dv, dvec
    return backward


def _decode_aligned_to_start(q, k, v, scale, causal):
    return ora.forward_rows(q, np.arange(np.shape(q)[0]), k, v, scale, causal)


def _backward_cross_aligned_to_start(q, k, v, do, scale, causal):
    return ora.backward(q, k, v, do, scale, causal)


def _merge_unweighted(o_parts, lse_parts):
    o, lse = _orig_merge(o_parts, lse_parts)
    return np.asarray(o_parts, float).mean(axis=0), lse


def _merge_lse_max(o_parts, lse_parts):
    o, lse = _orig_merge(o_parts, lse_parts)
    return o, np.asarray(lse_parts, float).max(axis=0)


_orig_merge = ora.merge_partials
_orig_scores = ora.scores
_orig_softmax = ora.softmax_rows

MUTANTS = {
    "scores_without_scale": ("scores", _scores_noscale),
    "scores_transposed": ("scores", _scores_transposed),
    "mask_wrong_direction": ("scores", _mask_variant(lambda j, i: j < i)),
    "mask_off_by_one": ("scores", _mask_variant(lambda j, i: j >= i)),
    "lse_without_log": ("softmax_rows", _softmax_no_log),
    "softmax_over_columns": ("softmax_rows", _softmax_columns),
    "output_uses_k": ("forward", _forward_uses_k),
    "backward_drops_D": ("backward", _backward_variant("drop_D")),
    "backward_sign_flip": ("backward", _backward_variant("flip_sign")),
    "backward_dq_without_scale": ("backward", _backward_variant("dq_noscale")),
    "backward_dk_untransposed": ("backward", _backward_variant("dk_untransposed")),
    "backward_dv_untransposed": ("backward", _backward_variant("dv_untransposed")),
    "decode_aligned_to_start": ("decode", _decode_aligned_to_start),
    "backward_cross_aligned_to_start": ("backward_cross", _backward_cross_aligned_to_start),
    "merge_unweighted": ("merge_partials", _merge_unweighted),
    "merge_lse_is_max": ("merge_partials", _merge_lse_max),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(ora)
        except Exception as e:  # a failed check or an error both expose the mistake
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_backward_copy_passes(monkeypatch):
    """The mutant template itself, without a mistake, passes every pin."""
    monkeypatch.setattr(ora, "backward", _backward_variant("none"))
    for pin in ALL_PINS:
        pin(ora)
