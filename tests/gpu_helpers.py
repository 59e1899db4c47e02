"""Helpers shared by the GPU parity tests: device upload, decode and the bars.

Bars (per element, GPU value upcast to fp64 minus the oracle's fp64 value):
  fp32 tensors   max |err| <= 1e-5
  bf16 tensors   |err| <= max(2e-2, ulp_bf16(ref)) per element and
                 mean |err| <= 2e-3
  LSE            |err| <= 1e-5 * max(1, |LSE|)   (relative, with an absolute
                 floor where LSE is near zero)

ulp_bf16(x) is the spacing of bfloat16 numbers at |x|: 2^(e - 7) for
2^e <= |x| < 2^(e + 1).  Below |x| = 4 it is at most 2^-6 < 2e-2, so the
absolute bar of 2e-2 applies unchanged; at |x| >= 4 the two bf16 neighbours of
the exact value are already 2^-5 = 0.031 apart and rounding the output to the
nearer one alone may cost 0.0156, so the element is allowed one spacing: half
for that final rounding, half for the bf16 rounding of the product operands (P,
dS) before it.  The mean bar is not widened.
"""
import sys

import numpy as np
import pytest
import torch

import synth

F32_MAX = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
LSE_REL = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """Upload a synth tensor: bf16 bit patterns become a bf16 tensor, fp32 stays fp32."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ulp_bf16(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits): 2^(e - 7) for
    2^e <= |x| < 2^(e + 1); the spacing of the smallest normals below them."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7.0)


def bf16_bar(ref):
    """Per-element max-error bar for bf16 outputs: max(2e-2, ulp_bf16(ref))."""
    return np.maximum(BF16_MAX, ulp_bf16(ref))


def check(got, ref, dtype, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_MAX, f"{what}: max abs err {err.max():.3e} > {F32_MAX}"
    else:
        over = err - bf16_bar(ref)
        i = int(np.argmax(over))
        assert over.max() <= 0, (f"{what}: abs err {err.flat[i]:.3e} at |ref| = {abs(ref.flat[i]):.3f} "
                                 f"above its bar {bf16_bar(ref).flat[i]:.3e}")
        assert err.mean() <= BF16_MEAN, f"{what}: mean abs err {err.mean():.3e} > {BF16_MEAN}"
    return float(err.max()), float(err.mean())


def dropout_d_terms(q, k, do, o_ref, scale, causal):
    """Bounds on how far the bf16 rounding of the stored O moves dQ and dK
    (fp64 arrays [N, d] of one head; o_ref the exact dropout output).

    The backward takes D_i = sum_c dO_ic O_ic from the O the forward stored in
    bf16, O_ic + e_ic with |e_ic| <= 2^-9 |O_ic| (round to nearest), so D_i
    is off by up to eps_i = 2^-9 sum_c |dO_ic| |O_ic|.  dS = P * (Z * dP - D)
    then carries -P_ij times that error: dQ_i moves by at most scale eps_i
    sum_j P_ij |K_j| and dK_j by at most scale sum_i P_ij eps_i |Q_i|.  Where
    a row sees few keys the exact dS is a small difference of large terms (a
    causal row that sees one key: s dP - D = 0 exactly), so this term can
    exceed the plain bars; without dropout such a row's O is a bf16 value of
    V and is stored exactly."""
    from oracle.attention import scores, softmax_rows   # test infrastructure only
    q, k, do, o_ref = (np.asarray(x, np.float64) for x in (q, k, do, o_ref))
    pm = softmax_rows(scores(q, k, scale, causal))[0]
    eps = 1.01 * 2.0 ** -9 * (np.abs(do) * np.abs(o_ref)).sum(axis=1)
    dq_term = abs(scale) * eps[:, None] * (pm @ np.abs(k))
    dk_term = abs(scale) * (pm.T @ (eps[:, None] * np.abs(q)))
    return dq_term, dk_term


def count_over(got, ref, bar=BF16_MAX):
    """Number of elements whose abs error exceeds `bar` (a report, not a check)."""
    return int((np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)) > bar).sum())


def check_lse(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert np.isfinite(got).all(), f"{what}: non-finite LSE"
    assert err.max() <= LSE_REL, f"{what}: LSE rel err {err.max():.3e} > {LSE_REL}"
    return float(err.max())


def check_dropout(got, ref, s, what, d_term=None):
    """Bar for outputs of the dropout entry points, s = the scale of kept
    probabilities: every kept term is multiplied by s, so outputs grow by up to
    s and so does the bf16 rounding of them (half an ulp is up to 2^-9 |x|).
    An element may differ from the oracle by 2^-8 |ref| (the rounding of the
    result, with margin) plus s times the plain path's absolute bar (2e-2),
    plus, for dQ and dK, `d_term` (dropout_d_terms: what the bf16 rounding
    of the stored O moves them by through D = rowsum(dO * O)); the mean error
    may reach s times the plain mean bar plus 2^-8 times the mean |ref|.  A
    wrong mask element moves a result by a whole term."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    over = err - 2.0 ** -8 * np.abs(ref) - (0.0 if d_term is None else d_term)
    assert over.max() <= BF16_MAX * s, f"{what}: max abs err {err.max():.3e} ({over.max():.3e} beyond 2^-8 |ref|)"
    mean_bar = BF16_MEAN * s + 2.0 ** -8 * np.abs(ref).mean()
    assert err.mean() <= mean_bar, f"{what}: mean abs err {err.mean():.3e} > {mean_bar:.2e}"


def inputs(shape, dtype, seed, with_do=False, qk_mult=1.0):
    host = synth.make_inputs(shape, dtype, seed, with_do=with_do, qk_mult=qk_mult)
    dev = {k: to_dev(v) for k, v in host.items()}
    f64 = {k: synth.decode(v) for k, v in host.items()}
    return dev, f64
