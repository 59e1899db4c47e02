"""Seeded synthetic inputs for exact scaled-dot-product attention.

This module is shared by the tests, the benchmark and the smoke check. It holds
the workload shapes and the random draws only, and none of the attention
arithmetic: neither the GPU path nor the CPU oracle depends on anything here
beyond the arrays it returns.

Workloads (all tensors use the [B, N, H, d] layout of the PyTorch module on the
page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org), section "代码手撕环节",
whose forward takes (batch, seq_len, num_heads, head_dim) tensors):

  c1  fp32 [1, 256, 1, 64]      non-causal, scale 1/8        forward only
  c2  bf16 [2, 512, 8, 64]      causal,     scale 1/8        forward only
                                (the usage example's shape on the same page)
  c3  bf16 [4, 4096, 16, 128]   non-causal and causal, scale fp32(1/sqrt(128))
  c4  bf16 [1, 32768, 32, 128]  causal, Q and K doubled after rounding
  c5  bf16 [2, 8192, 16, 64]    causal, scale 1/8, forward + backward (with dO)

Values are i.i.d. standard normal, drawn with numpy's PCG64 generator seeded
with the workload number, in the order Q, K, V, dO, as float32 and then rounded
to bfloat16 with round-to-nearest-even.  The bf16 tensors are returned as their
raw uint16 bit patterns so that the GPU and the oracle consume the same bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                  # "bf16" or "f32"
    scale: float                # the float32 value passed to the kernels
    causal: tuple               # which mask settings the workload runs
    seed: int
    backward: bool = False
    qk_mult: float = 1.0        # exact power-of-two factor applied to Q and K
    check_heads: int = 0        # 0: every (b, h); else this many seeded heads
    check_rows: int = 0         # 0: every row; else this many seeded rows per head
    note: str = field(default="", compare=False)

    @property
    def shape(self):
        return (self.B, self.N, self.H, self.d)


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 value (returned as float)."""
    return float(np.float32(x))


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 64, "f32", f32(1 / math.sqrt(64)), (False,), seed=1),
    "c2": Workload("c2", 2, 8, 512, 64, "bf16", 0.125, (True,), seed=2),
    "c3": Workload("c3", 4, 16, 4096, 128, "bf16", f32(1 / math.sqrt(128)), (False, True), seed=3,
                   check_heads=2),
    "c4": Workload("c4", 1, 32, 32768, 128, "bf16", f32(1 / math.sqrt(128)), (True,), seed=4,
                   qk_mult=2.0, check_rows=512),
    "c5": Workload("c5", 2, 16, 8192, 64, "bf16", 0.125, (True,), seed=5, backward=True,
                   check_heads=2),
}


# --------------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  NaN is not expected from the generators
    and is not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of a tensor returned by :func:`make_inputs`."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------- draws

def draw(shape, dtype: str, rng: np.random.Generator, mult: float = 1.0) -> np.ndarray:
    """One standard-normal tensor: float32 for "f32", bf16 bits for "bf16"."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x * np.float32(mult)
    bits = f32_to_bf16_bits(x)
    if mult != 1.0:
        # Power-of-two factors are exact on bf16 values, so scaling after rounding
        # keeps the tensor a set of bf16 values.
        bits = f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(mult))
    return bits


def make_inputs(shape, dtype: str, seed: int, with_do: bool = False, qk_mult: float = 1.0) -> dict:
    """Seeded Q, K, V (and dO) of the given [B, N, H, d] shape, in that draw order."""
    rng = np.random.default_rng(seed)
    out = {
        "q": draw(shape, dtype, rng, qk_mult),
        "k": draw(shape, dtype, rng, qk_mult),
        "v": draw(shape, dtype, rng),
    }
    if with_do:
        out["do"] = draw(shape, dtype, rng)
    return out


def make_decode_inputs(B: int, Nq: int, Nk: int, H: int, d: int, seed: int, qk_mult: float = 1.0,
                       with_do: bool = False) -> dict:
    """Seeded Q ([B, Nq, H, d]), K and V ([B, Nk, H, d]) and, with with_do, dO
    ([B, Nq, H, d]) as bf16 bits, in that draw order."""
    rng = np.random.default_rng(seed)
    out = {
        "q": draw((B, Nq, H, d), "bf16", rng, qk_mult),
        "k": draw((B, Nk, H, d), "bf16", rng, qk_mult),
        "v": draw((B, Nk, H, d), "bf16", rng),
    }
    if with_do:
        out["do"] = draw((B, Nq, H, d), "bf16", rng)
    return out


def to_e4m3(x: np.ndarray):
    """Per-tensor e4m3 quantisation of float32 values: the descale maps max |x|
    to 448 (the largest e4m3 magnitude), codes are x / descale rounded to
    nearest even by torch's float8_e4m3fn conversion.  Returns (codes as
    uint8, descale as a float32 value)."""
    import torch
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = f32(amax / 448.0) if amax > 0 else 1.0
    y = torch.from_numpy(np.ascontiguousarray(x / np.float32(descale), dtype=np.float32))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), descale


def make_fp8_inputs(B: int, Nq: int, Nk: int, H: int, d: int, seed: int, sink: float = 0.0,
                    qk_int: bool = False) -> dict:
    """Seeded e4m3 Q ([B, Nq, H, d]), K and V ([B, Nk, H, d]) with their descales.

    Q, K, V are drawn as float32 standard normals in that order and quantised
    per tensor (to_e4m3).  qk_int: Q and K become the integers
    clip(rint(4 x), -15, 15) with descale 1/4 instead (every such integer is
    an e4m3 value, and the scores are sums of integer products).  sink > 0
    adds an attention-sink key: the last feature of every query is 2, that of
    key 0 is `sink` and that of every other key 0 (before quantisation).
    Returns {"q", "k", "v": uint8 codes, "descales": (dq, dk, dv)}."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Nq, H, d), dtype=np.float32)
    k = rng.standard_normal((B, Nk, H, d), dtype=np.float32)
    v = rng.standard_normal((B, Nk, H, d), dtype=np.float32)
    if sink > 0:
        q[..., d - 1] = 2.0
        k[..., d - 1] = 0.0
        k[:, 0, :, d - 1] = sink
    if qk_int:
        import torch

        def ints(x):
            t = torch.from_numpy(np.clip(np.rint(4 * x), -15, 15).astype(np.float32))
            return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        q8, k8, dq, dk = ints(q), ints(k), 0.25, 0.25
    else:
        (q8, dq), (k8, dk) = to_e4m3(q), to_e4m3(k)
    v8, dv = to_e4m3(v)
    return {"q": q8, "k": k8, "v": v8, "descales": (dq, dk, dv)}


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.shape, w.dtype, w.seed, with_do=w.backward, qk_mult=w.qk_mult)


def checked_heads(w: Workload) -> list:
    """The (b, h) pairs the oracle checks: all of them, or a seeded draw."""
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    if not w.check_heads:
        return pairs
    rng = np.random.default_rng(w.seed + 100)
    idx = rng.choice(len(pairs), size=w.check_heads, replace=False)
    return [pairs[i] for i in sorted(idx)]


def checked_rows(w: Workload, h: int) -> np.ndarray:
    """Query rows checked for head h: all, or a seeded draw that keeps 0 and N-1."""
    if not w.check_rows:
        return np.arange(w.N)
    rng = np.random.default_rng(w.seed + 200 + h)
    inner = rng.choice(np.arange(1, w.N - 1), size=w.check_rows - 2, replace=False)
    return np.sort(np.concatenate([[0, w.N - 1], inner])).astype(np.int64)
