"""Seeded random sweep of every entry point against the fp64 oracle.

Forty configurations drawn from one seeded generator: batch, heads, ragged
lengths (uniform, or one off a multiple of 64), head size, mask, scale
(d^-0.5 times a factor in [1/2, 2]), and per entry point its own parameters
(key length of the cross forms, query rows of the decode, p, seed and offset
of the dropout).  Up to four heads of each configuration (the first, the
last and two drawn) are compared with the oracle under the same bars as the
dedicated tests: `check` / `check_lse` (bf16, fp32), `check_dropout`, and the
FP8 rounding bound of `fp8_bounds`.  The configurations are fixed by the seed,
not chosen after a run.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.attention as ora
import oracle.dropout as drop
import oracle.fp8 as fp8
import synth
from fp8_bounds import loose_bound, lse_bound
from gpu_helpers import check, check_dropout, check_lse, dropout_d_terms, require_gpu, say, to64, to_dev

pytestmark = pytest.mark.gpu

KINDS = ("square", "cross", "decode", "dropout", "f32", "fp8")
HEAD_SIZES = {"square": (64, 128, 256), "cross": (64, 128, 256), "decode": (64, 128),
              "dropout": (64, 128, 256), "f32": (64, 128), "fp8": (64, 128)}


def _length(rng, hi):
    if rng.random() < 0.4:
        return int(max(1, min(hi, 64 * rng.integers(1, hi // 64 + 1) + rng.integers(-1, 2))))
    return int(rng.integers(1, hi + 1))


def _configs(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = KINDS[i % len(KINDS)]
        d = int(rng.choice(HEAD_SIZES[kind]))
        c = {"kind": kind, "B": int(rng.integers(1, 4)), "H": int(rng.choice([1, 2, 3, 5])), "d": d,
             "causal": bool(rng.random() < 0.5), "mult": float(2.0 ** rng.uniform(-1, 1)),
             "seed": int(rng.integers(1, 2 ** 31))}
        if kind == "decode":
            c["Nq"], c["Nk"] = int(rng.integers(1, 33)), _length(rng, 3000)
            if c["causal"]:
                c["Nk"] = max(c["Nk"], c["Nq"])      # causal rows are the last Nq of Nk positions
        elif kind in ("cross", "fp8"):
            c["Nq"], c["Nk"] = _length(rng, 600), _length(rng, 900)
            if c["causal"] and c["Nq"] > c["Nk"]:
                c["Nq"], c["Nk"] = c["Nk"], c["Nq"]
        else:
            c["Nq"] = c["Nk"] = _length(rng, 700)
        if kind == "dropout":
            c["p"] = float(rng.uniform(0.05, 0.6))
            c["dseed"], c["offset"] = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 31))
        out.append(c)
    return out


CONFIGS = _configs()


def _heads(c):
    rng = np.random.default_rng(c["seed"])
    all_heads = [(b, h) for b in range(c["B"]) for h in range(c["H"])]
    pick = {all_heads[0], all_heads[-1]}
    for i in rng.choice(len(all_heads), size=min(2, len(all_heads)), replace=False):
        pick.add(all_heads[int(i)])
    return sorted(pick)


def _label(c):
    return "-".join(f"{k}{c[k]}" for k in ("kind", "B", "Nq", "Nk", "H", "d", "causal"))


@pytest.mark.parametrize("c", CONFIGS, ids=_label)
def test_sweep(c):
    require_gpu()
    kind, B, H, d, causal = c["kind"], c["B"], c["H"], c["d"], c["causal"]
    Nq, Nk = c["Nq"], c["Nk"]
    scale = synth.f32(c["mult"] * d ** -0.5)
    say("sweep", _label(c), f"scale={scale:.4f}", {k: c[k] for k in ("p", "offset") if k in c})
    if kind == "fp8":
        host = synth.make_fp8_inputs(B, Nq, Nk, H, d, seed=c["seed"])
        q, k, v = (torch.from_numpy(np.ascontiguousarray(host[x])).cuda().view(torch.float8_e4m3fn) for x in "qkv")
        o, lse = fa.forward_fp8(q, k, v, descales=host["descales"], scale=scale, causal=causal)
        torch.cuda.synchronize()
        o64, l64 = to64(o), to64(lse)
        for b, h in _heads(c):
            q8, k8, v8 = host["q"][b, :, h], host["k"][b, :, h], host["v"][b, :, h]
            o_ex, lse_ex = fp8.forward(q8, k8, v8, *host["descales"], scale, causal)
            assert np.isfinite(o64[b, :, h]).all()
            err = np.abs(o64[b, :, h] - o_ex)
            lb = loose_bound(q8, k8, v8, host["descales"], scale, causal, o_ex)
            assert (err <= lb).all(), f"fp8 O (b={b}, h={h}) outside its bound by {(err - lb).max():.3e}"
            lerr = np.abs(l64[b, h] - lse_ex)
            assert (lerr <= lse_bound(q8, k8, host["descales"], scale, causal, lse_ex)).all(), "fp8 LSE"
        return
    dtype = "f32" if kind == "f32" else "bf16"
    if kind in ("cross", "decode"):
        host = synth.make_decode_inputs(B, Nq, Nk, H, d, seed=c["seed"], with_do=(kind == "cross"))
    else:
        host = synth.make_inputs((B, Nq, H, d), dtype, c["seed"], with_do=True)
    dev = {x: to_dev(a) for x, a in host.items()}
    f64 = {x: synth.decode(a) for x, a in host.items()}
    grads = None
    if kind == "decode":
        o, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal)
    elif kind == "cross":
        o, lse = fa.forward_cross(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal)
        grads = fa.backward_cross(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=scale, causal=causal)
    elif kind == "dropout":
        o, lse = fa.forward_dropout(dev["q"], dev["k"], dev["v"], c["p"], c["dseed"], c["offset"],
                                    scale=scale, causal=causal)
        grads = fa.backward_dropout(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, c["p"], c["dseed"],
                                    c["offset"], scale=scale, causal=causal)
    else:
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal)
        grads = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    g64 = [to64(g) for g in grads] if grads is not None else None
    for b, h in _heads(c):
        qh, kh, vh = (f64[x][b, :, h] for x in "qkv")
        what = f"{kind} (b={b}, h={h})"
        if kind == "dropout":
            keep = drop.keep_mask(b * H + h, np.arange(Nq), Nk, c["p"], c["dseed"], c["offset"])
            o_r, lse_r = drop.forward(qh, kh, vh, scale, causal, keep, c["p"])
            refs = drop.backward(qh, kh, vh, f64["do"][b, :, h], scale, causal, keep, c["p"])[:3]
            s = drop.keep_scale(c["p"])
            check_dropout(o64[b, :, h], o_r, s, f"O {what}")
            terms = dropout_d_terms(qh, kh, f64["do"][b, :, h], o_r, scale, causal) + (None,)
            for name, g, r, t in zip(("dQ", "dK", "dV"), g64, refs, terms):
                check_dropout(g[b, :, h], r, s, f"{name} {what}", t)
        else:
            if kind in ("cross", "decode"):
                o_r, lse_r = ora.decode(qh, kh, vh, scale, causal)
            else:
                o_r, lse_r = ora.forward(qh, kh, vh, scale, causal)
            check(o64[b, :, h], o_r, dtype, f"O {what}")
            if g64 is not None:
                if kind == "cross":
                    refs = ora.backward_cross(qh, kh, vh, f64["do"][b, :, h], scale, causal)[:3]
                else:
                    refs = ora.backward(qh, kh, vh, f64["do"][b, :, h], scale, causal)[:3]
                for name, g, r in zip(("dQ", "dK", "dV"), g64, refs):
                    check(g[b, :, h], r, dtype, f"{name} {what}")
        check_lse(l64[b, h], lse_r, f"LSE {what}")
