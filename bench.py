#!/usr/bin/env python3
"""Throughput of the fused exact-attention hot path on one MI355X.

One step = one forward (fa_forward) and one backward (fa_backward_preprocess
then fa_backward_dqdkdv - exactly what fa_backward runs) of bf16
causal attention on the forward+backward workload [B, N, H, d] = [2, 8192, 16,
64], scale 1/8, inputs seeded N(0, 1) and already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line.  value = credited TFLOP/s of the whole step, with the
forward credited 4 B H N^2 d / 2 FLOPs (causal) and the backward 2.5 times
that.  `roofline` covers the kernel with the largest average duration,
timed with HIP events recorded around each launch on the stream the kernels
run on.  `cpu_baseline` times the fp64 CPU oracle on one head of the same
workload.  `forward_only` times the forward alone on the two long causal
workloads ([4, 4096, 16, 128] and [1, 32768, 32, 128] with Q, K doubled);
`head256` times fa_forward and fa_backward at head size 256 ([2, 4096, 16,
256], causal and not); `library_gemm` times the vendor library's square
8192 GEMM in bf16 and e4m3 on the same device, as context for the spec peaks.

    python bench.py --copy-calibration

runs only a plain device copy of 256 MiB (for scaling hardware byte counters).

    python bench.py --kernel-case {c5,c3_causal,c3_noncausal,c4,c2,h256_causal} [--steps K]

runs only that workload's launches (c5: the forward + backward step;
h256_causal: fa_forward and fa_backward at [2, 4096, 16, 256] causal; the
others: the forward), for profiling one kernel under rocprofv3.

Besides the back-to-back timing that gives `value`, the line carries per-kernel
median, p10 and p90 of the same launches, a cold-cache timing of the step (a
512 MiB buffer, twice the 256 MB Infinity Cache, is written before each step),
the shader clock measured while the step runs, and the host's core counts
beside the CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2      # 256 CU x 2.4 GHz x 8192 dense e4m3 FLOP/clk/CU
PEAK_FP32_MATRIX_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s (bf16 fwd & fwd+bwd, causal) and % of MI355X MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, H, N, d, causal):
    return 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)


def copy_calibration():
    import torch
    n = 256 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 launches, each reads {n * 4} B and writes {n * 4} B")


# counter summary of each kernel of the c5 step (profiles/)
COUNTER_FILES = {"fwd": "counters_fwd_d64_causal.md", "bwd_dqdkdv": "counters_bwd_dqdkdv.md",
                 "bwd_preprocess": "counters_bwd_preprocess.md"}


def kernel_traffic(name):
    """HBM bytes per launch (TCC read and write request counts, copy-calibrated)
    from the committed counter summary, if it matches the current source."""
    if name not in COUNTER_FILES:
        return None
    path = os.path.join(ROOT, "profiles", COUNTER_FILES[name])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    src = re.search(r"source_file:\s*(\S+)", text)
    if not (m and h and src):
        return None
    cur = hashlib.sha256(open(os.path.join(ROOT, src.group(1)), "rb").read()).hexdigest()
    return float(m.group(1)) if cur == h.group(1) else None


def warm_up(fn, torch, min_seconds=0.2):
    """Untimed launches for at least `min_seconds` of wall time: after an idle
    gap (the CPU baseline, tensor set-up) the shader clock needs load to come
    back up, and a fixed count of short launches does not give it enough."""
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_seconds:
            return


def pct(xs, q):
    """q-quantile of a list (nearest rank)."""
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def stats_ms(xs):
    return {"median": round(pct(xs, 0.5), 4), "p10": round(pct(xs, 0.1), 4), "p90": round(pct(xs, 0.9), 4),
            "mean": round(sum(xs) / len(xs), 4)}


def sclk_under_load(step, torch, cycles=20_000_000, load_steps=25):
    """Shader clock (MHz) while `step` runs.  A one-wave spin of a fixed
    number of shader-clock cycles (torch.cuda._sleep, which counts the
    shader clock) runs on a second stream of default priority while the main
    stream runs `load_steps` steps before and after it; cycles / elapsed time
    of the spin, between events on its own stream, is the clock under that
    load.  The same spin on an idle GPU gives the clock at low load."""
    side = torch.cuda.Stream()
    out = {}
    for name, load in (("idle", 0), ("under_load", load_steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(load):
            step()
        with torch.cuda.stream(side):
            e0.record(side)
            torch.cuda._sleep(cycles)
            e1.record(side)
        for _ in range(load):
            step()
        torch.cuda.synchronize()
        out[name] = round(cycles / (e0.elapsed_time(e1) * 1e-3) / 1e6, 1)
    out["source"] = ("a spin of %d shader-clock cycles (torch.cuda._sleep) on a side stream, timed with "
                     "events, alone and beside %d fwd+bwd steps on each side" % (cycles, load_steps))
    return out


def host_cores():
    """os.cpu_count(), the affinity mask's size and the BLAS thread count."""
    blas = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas_threads": blas}


def time_forward_only(fa, torch, B, N, H, d, scale, qk_mult, seed, iters, causal=True):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32) * qk_mult).to(torch.bfloat16)
    k = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32) * qk_mult).to(torch.bfloat16)
    v = torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    warm_up(lambda: fa.fa_forward(q, k, v, o, lse, scale, causal), torch)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(st)
    for i in range(iters):
        fa.fa_forward(q, k, v, o, lse, scale, causal)
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    med = ms[len(ms) // 2]
    tf = fwd_flops(B, H, N, d, causal) / (med * 1e-3) / 1e12
    del q, k, v, o, lse
    return {"shape_BNHd": [B, N, H, d], "causal": causal, "median_ms": round(med, 4),
            "p10_ms": round(pct(ms, 0.1), 4), "p90_ms": round(pct(ms, 0.9), 4),
            "tflops": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}


def time_forward_fp8(fa, torch, B, N, H, d, seed, iters, causal=True, qk_mult=1.0):
    """fa_forward_fp8 on e4m3 inputs (standard normal draws quantised per
    tensor, the descale mapping max |x| to 448): median call time (the V^T
    pre-pass and the forward) and its rate against the FP8 matrix peak."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    xs, descales = [], []
    for mult in (qk_mult, qk_mult, 1.0):
        x = torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32) * mult
        ds = float(x.abs().max()) / 448.0
        xs.append((x / ds).to(torch.float8_e4m3fn))
        descales.append(ds)
        del x
    q, k, v = xs
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_forward_fp8_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    scale = d ** -0.5
    call = lambda: fa.fa_forward_fp8(q, k, v, *descales, o, lse, ws, scale, causal)  # noqa: E731
    warm_up(call, torch)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(st)
    for i in range(iters):
        call()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    med = ms[len(ms) // 2]
    tf = fwd_flops(B, H, N, d, causal) / (med * 1e-3) / 1e12
    del q, k, v, o, lse, ws
    return {"shape_BNHd": [B, N, H, d], "causal": causal, "median_ms": round(med, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)}}


def time_fp32(fa, torch, B, N, H, d, causal, iters):
    """fa_forward_f32 and fa_backward_f32 (fp32 tensors, fp32 matrix cores):
    median times, and rates against the fp32 matrix peak (the backward at the
    credited 2.5x forward FLOPs)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    calls = {"fwd": lambda: fa.fa_forward(q, k, v, o, lse, scale, causal),
             "bwd": lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws, scale, causal)}
    out = {"shape_BNHd": [B, N, H, d], "causal": causal}
    st = torch.cuda.current_stream()
    for name, call in calls.items():
        warm_up(call, torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(st)
        for i in range(iters):
            call()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
        med = ms[len(ms) // 2]
        tf = (1.0 if name == "fwd" else 2.5) * fwd_flops(B, H, N, d, causal) / (med * 1e-3) / 1e12
        out[name] = {"median_ms": round(med, 4), "tflops": round(tf, 2),
                     "pct_of_fp32_matrix_peak": round(100 * tf / PEAK_FP32_MATRIX_TFLOPS, 1)}
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def time_library_gemm(torch, n, iters=10):
    """The vendor library's square GEMM (torch.matmul on bf16, torch._scaled_mm
    on e4m3) on the same device: the rate a plain dense contraction reaches
    under the same clock and power limits, reported beside the spec peaks."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    out = {"n": n}
    one = torch.tensor(1.0, device="cuda")
    a8 = a.to(torch.float8_e4m3fn)
    b8 = b.to(torch.float8_e4m3fn).t().contiguous().t()   # column-major, as _scaled_mm takes it
    calls = {"bf16": (lambda: a @ b, PEAK_BF16_TFLOPS),
             "fp8_e4m3": (lambda: torch._scaled_mm(a8, b8, one, one, out_dtype=torch.bfloat16), PEAK_FP8_TFLOPS)}
    st = torch.cuda.current_stream()
    for name, (fn, peak) in calls.items():
        try:
            warm_up(fn, torch)
        except Exception as e:   # an op this torch build does not provide
            out[name] = {"error": str(e)[:120]}
            continue
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(st)
        for i in range(iters):
            fn()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
        med = ms[len(ms) // 2]
        tf = 2 * n ** 3 / (med * 1e-3) / 1e12
        out[name] = {"median_ms": round(med, 4), "tflops": round(tf, 1), "pct_of_peak": round(100 * tf / peak, 1)}
    del a, b, a8, b8
    return out


def time_fwd_bwd(fa, torch, B, N, H, d, causal, iters):
    """fa_forward and fa_backward (preprocess + both passes) timed apart:
    medians and the rates at 4 B H N^2 d (halved under the mask) and 2.5x
    that."""
    g = torch.Generator(device="cuda")
    g.manual_seed(10)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    scale = d ** -0.5
    calls = {"fwd": lambda: fa.fa_forward(q, k, v, o, lse, scale, causal),
             "bwd": lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws, scale, causal)}
    out = {"shape_BNHd": [B, N, H, d], "causal": causal}
    st = torch.cuda.current_stream()
    for name, fn in calls.items():
        warm_up(fn, torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(st)
        for i in range(iters):
            fn()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
        med = ms[len(ms) // 2]
        tf = (1.0 if name == "fwd" else 2.5) * fwd_flops(B, H, N, d, causal) / (med * 1e-3) / 1e12
        out[name] = {"median_ms": round(med, 4), "p10_ms": round(pct(ms, 0.1), 4), "p90_ms": round(pct(ms, 0.9), 4),
                     ("tflops" if name == "fwd" else "tflops_credited"): round(tf, 1),
                     "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def time_dropout(fa, torch, B, N, H, d, p, iters):
    """fa_forward_dropout + fa_backward_dropout (causal): median step time and
    the rate at the FLOPs credited to the plain step (dropout adds none)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    scale = d ** -0.5

    def step():
        fa.fa_forward_dropout(q, k, v, o, lse, scale, True, p, 1234, 0)
        fa.fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, scale, True, p, 1234, 0)
    warm_up(step, torch)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(st)
    for i in range(iters):
        step()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    med = ms[len(ms) // 2]
    tf = 3.5 * fwd_flops(B, H, N, d, True) / (med * 1e-3) / 1e12
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return {"shape_BNHd": [B, N, H, d], "causal": True, "p_drop": p, "median_step_ms": round(med, 4),
            "tflops_credited": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}


def time_single_pass(fa, torch, B, N, H, d, iters):
    """fa_backward_single_pass (causal; zeroing of the dQ accumulator, the
    preprocess, the dK/dV pass with atomic dQ, the dQ conversion) against
    fa_backward on the same inputs: median call times and the backward's
    credited rate (2.5x the forward's FLOPs)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, scale=scale, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws1 = torch.empty(fa.fa_backward_single_pass_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32,
                      device="cuda")
    ws2 = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    calls = {"single_pass": lambda: fa.fa_backward_single_pass(q, k, v, o, do, lse, dq, dk, dv, ws1, scale, True),
             "two_pass": lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws2, scale, True)}
    out = {"shape_BNHd": [B, N, H, d], "causal": True}
    st = torch.cuda.current_stream()
    for name, fn in calls.items():
        warm_up(fn, torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(st)
        for i in range(iters):
            fn()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
        med = ms[len(ms) // 2]
        tf = 2.5 * fwd_flops(B, H, N, d, True) / (med * 1e-3) / 1e12
        out[name] = {"median_ms": round(med, 4), "tflops_credited": round(tf, 1),
                     "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)}
    del q, k, v, do, o, lse, dq, dk, dv, ws1, ws2
    return out


def time_decode(fa, torch, B, Nq, Nk, H, d, seed, iters):
    """Split-key decode of Nq rows against a [B, Nk, H, d] K/V cache (causal, the
    rows being the last Nq positions): median launch pair (split + merge) time and
    the HBM roofline of reading K and V once."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((B, Nq, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, Nk, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, Nk, H, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    splits = fa.fa_decode_splits(B, H, Nq, Nk, d)
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits) // 4, dtype=torch.float32,
                     device="cuda")
    scale = d ** -0.5
    warm_up(lambda: fa.fa_decode(q, k, v, o, lse, ws, scale, True, splits), torch)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(st)
    for i in range(iters):
        fa.fa_decode(q, k, v, o, lse, ws, scale, True, splits)
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(iters))
    med = ms[len(ms) // 2]
    alg = 2.0 * B * Nk * H * d * 2 + 2.0 * B * Nq * H * d * 2 + 4.0 * B * H * Nq
    gbs = alg / (med * 1e-3) / 1e9
    del q, k, v, o, lse, ws
    return {"shape_B_Nq_Nk_H_d": [B, Nq, Nk, H, d], "causal": True, "splits": splits,
            "median_ms": round(med, 4), "algorithmic_bytes": alg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def cpu_baseline(w, host, got, min_seconds=10.0):
    """Time the fp64 oracle (forward + backward) on whole heads of the workload,
    head after head, until at least `min_seconds` of CPU work; also compare the
    first head with the GPU results."""
    import numpy as np
    import oracle.attention as ora
    import synth
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=1)
    except Exception:   # threadpoolctl missing: fall back to the affinity mask
        threads = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    errs, done, dt = {}, 0, 0.0
    for b, h in heads:
        q, k, v, do = (synth.decode(host[n][b, :, h]) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        o_ref, lse_ref = ora.forward(q, k, v, w.scale, True)
        dq_ref, dk_ref, dv_ref, _ = ora.backward(q, k, v, do, w.scale, True)
        dt += time.perf_counter() - t0
        done += 1
        if done == 1:
            for name, ref in (("O", o_ref), ("dQ", dq_ref), ("dK", dk_ref), ("dV", dv_ref)):
                g = got[name][b, :, h].float().cpu().numpy().astype(np.float64)
                errs[name] = float(np.abs(g - ref).max())
            lg = got["LSE"][b, h].cpu().numpy().astype(np.float64)
            errs["LSE_rel"] = float(np.max(np.abs(lg - lse_ref) / np.maximum(1, np.abs(lse_ref))))
        if dt >= min_seconds:
            break
    flops = fwd_flops(1, 1, w.N, w.d, True) * 3.5 * done
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 numpy oracle, forward + backward of {done} whole head(s) of the same workload "
                   f"(N={w.N}, d={w.d}, causal) in {dt:.1f} s; credited FLOPs as for the GPU"),
        "seconds": round(dt, 2), "host": host_cores(),
    }, errs


def kernel_case(fa, torch, synth, name, steps):
    """Launches of one workload only (for profiling one kernel): `steps`
    launches after a time-based warm-up; prints a short line."""
    cases = {
        "c3_causal": (4, 4096, 16, 128, True, 1.0, 3),
        "c3_noncausal": (4, 4096, 16, 128, False, 1.0, 3),
        "c4": (1, 32768, 32, 128, True, 2.0, 4),
        "c2": (2, 512, 8, 64, True, 1.0, 2),
    }
    if name == "h256_causal":
        # fa_forward then fa_backward (preprocess + the fused grid) on
        # [2, 4096, 16, 256] causal, as in the line's head256 block.
        r = time_fwd_bwd(fa, torch, 2, 4096, 16, 256, True, steps)
        print(json.dumps({"kernel_case": name, **r}), flush=True)
        return
    B, N, H, d, causal, mult, seed = cases[name]
    r = time_forward_only(fa, torch, B, N, H, d, synth.f32(d ** -0.5) if d != 64 else 0.125, mult, seed, steps,
                          causal=causal)
    print(json.dumps({"kernel_case": name, **r}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kernel-case", choices=["c5", "c3_causal", "c3_noncausal", "c4", "c2", "h256_causal"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (heads would shard "
              "across GPUs with no communication, each running these kernels on its share); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import exact_io_aware_39_amd as fa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.kernel_case and args.kernel_case != "c5":
        kernel_case(fa, torch, synth, args.kernel_case, args.steps)
        return

    w = synth.WORKLOADS["c5"]
    B, N, H, d = w.shape
    log(f"bench: workload c5 [B,N,H,d]={list(w.shape)} bf16 causal scale={w.scale}")
    host = synth.workload_inputs(w)
    dev = {k: torch.from_numpy(v.view(np.int16)).cuda().view(torch.bfloat16) for k, v in host.items()}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(st)
        fa.fa_forward(q, k, v, o, lse, w.scale, True)
        if evs:
            evs[1].record(st)
        fa.fa_backward_preprocess(o, do, lse, ws)
        if evs:
            evs[2].record(st)
        fa.fa_backward_dqdkdv(q, k, v, do, ws, dq, dk, dv, w.scale, True)
        if evs:
            evs[3].record(st)

    if args.kernel_case == "c5":
        warm_up(step, torch)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"kernel_case": "c5", "steps": args.steps}), flush=True)
        return

    names = ["fwd", "bwd_preprocess", "bwd_dqdkdv"]
    # Warm-up: the requested count, and at least 0.2 s of load so that the
    # shader clock has come up before the timed steps.
    for _ in range(args.warmup):
        step()
    warm_up(step, torch)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]
           for j, n in enumerate(names)}
    # Cold caches: before each step, write 512 MiB (twice the Infinity
    # Cache) so that no input of the step is left in L2 or MALL.
    ncold = min(args.steps, 20)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(ncold)]
    for i in range(ncold):
        flush.fill_(float(i))
        step(cold_ev[i])
    torch.cuda.synchronize()
    cold = {n: [cold_ev[i][j].elapsed_time(cold_ev[i][j + 1]) for i in range(ncold)]
            for j, n in enumerate(names)}
    cold_step = [cold_ev[i][0].elapsed_time(cold_ev[i][3]) for i in range(ncold)]
    del flush
    avg = {n: sum(x) / len(x) for n, x in per.items()}
    ms_step = wall * 1e3 / args.steps

    F = fwd_flops(B, H, N, d, True)
    Fb = 2.5 * F
    value = (F + Fb) / (ms_step * 1e-3) / 1e12
    fwd_ms = avg["fwd"]
    bwd_ms = avg["bwd_preprocess"] + avg["bwd_dqdkdv"]
    pairs = B * H * N * N / 2.0                      # visible (query, key) pairs, causal
    alg = {   # algorithmic work of one launch of each kernel
        "fwd": ("mfma", 4.0 * d * pairs),            # S = QK^T and O += PV
        # the backward is credited 2.5x the forward (five N x N x d products);
        # the two-pass kernel also recomputes S and dP once more in its dQ
        # tiles, which is reported separately as executed work
        "bwd_dqdkdv": ("mfma", 10.0 * d * pairs),
        "bwd_preprocess": ("hbm", 2.0 * B * N * H * d * 2 + 12.0 * B * H * N),  # read O, dO, LSE; write D, -LSE log2 e
    }
    executed = {"fwd": 4.0 * d * pairs, "bwd_dqdkdv": 14.0 * d * pairs}
    dom = max(avg, key=avg.get)
    bound, work = alg[dom]
    if bound == "mfma":
        achieved = work / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = work / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(achieved / roof["peak"], 4)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(avg[dom], 4)
    roof["algorithmic_per_launch"] = work
    if dom in executed:
        roof["executed_mfma_tflops"] = round(executed[dom] / (avg[dom] * 1e-3) / 1e12, 1)
    roof["traffic"] = kernel_traffic(dom)
    sclk = sclk_under_load(step, torch)
    if bound == "mfma" and sclk.get("under_load"):
        # the same launch against the MFMA rate at the clock observed under this load
        roof["frac_at_observed_sclk"] = round(achieved / (PEAK_BF16_TFLOPS * sclk["under_load"] / 2400.0), 4)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fwd+bwd causal bf16 [B,N,H,d]=[2,8192,16,64], scale 1/8, seeded N(0,1)",
                   "B": B, "N": N, "H": H, "d": d, "causal": True, "scale": w.scale},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "breakdown": {
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_tflops": round(F / (fwd_ms * 1e-3) / 1e12, 1),
            "bwd_tflops_credited": round(Fb / (bwd_ms * 1e-3) / 1e12, 1),
            "fwd_pct_of_peak": round(100 * F / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "bwd_pct_of_peak_credited": round(100 * Fb / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernel_avg_ms": {n: round(x, 4) for n, x in avg.items()},
            "kernel_ms": {n: stats_ms(x) for n, x in per.items()},
        },
        "cold_cache": {
            "note": "512 MiB written before each step (caches cold); per-kernel times in ms",
            "steps": ncold, "step_ms": stats_ms(cold_step),
            "kernel_ms": {n: stats_ms(x) for n, x in cold.items()},
            "fwd_pct_of_peak": round(100 * F / (pct(cold["fwd"], 0.5) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "bwd_pct_of_peak_credited": round(100 * Fb / ((pct(cold["bwd_preprocess"], 0.5)
                                                           + pct(cold["bwd_dqdkdv"], 0.5)) * 1e-3)
                                              / 1e12 / PEAK_BF16_TFLOPS, 2),
        },
        "sclk": sclk,
        "host": host_cores(),
    }

    if not args.no_extra:
        log("bench: forward-only workloads")
        result["forward_only"] = {
            "c2": time_forward_only(fa, torch, 2, 512, 8, 64, 0.125, 1.0, 2, 50),
            "c3_causal": time_forward_only(fa, torch, 4, 4096, 16, 128, synth.f32(128 ** -0.5), 1.0, 3, 20),
            "c3_noncausal": time_forward_only(fa, torch, 4, 4096, 16, 128, synth.f32(128 ** -0.5), 1.0, 3, 20,
                                              causal=False),
            "c4": time_forward_only(fa, torch, 1, 32768, 32, 128, synth.f32(128 ** -0.5), 2.0, 4, 10),
        }
        result["forward_only"]["c2"]["note"] = "reported, not targeted (64 workgroups for 256 CUs)"
        log("bench: library GEMM on the same device")
        result["library_gemm"] = time_library_gemm(torch, 8192)
        result["library_gemm"]["note"] = ("vendor GEMM (hipBLASLt through torch), context for the spec peaks; "
                                          "not part of value")
        log("bench: head size 256")
        result["head256"] = {
            "causal": time_fwd_bwd(fa, torch, 2, 4096, 16, 256, True, 20),
            "noncausal": time_fwd_bwd(fa, torch, 2, 4096, 16, 256, False, 10),
        }
        log("bench: FP8 (e4m3) forward")
        result["forward_fp8"] = {
            "c3_causal": time_forward_fp8(fa, torch, 4, 4096, 16, 128, 3, 20),
            "c3_noncausal": time_forward_fp8(fa, torch, 4, 4096, 16, 128, 3, 20, causal=False),
            "c4": time_forward_fp8(fa, torch, 1, 32768, 32, 128, 4, 10, qk_mult=2.0),
        }
        log("bench: fp32 path (fp32 matrix cores)")
        result["fp32"] = {
            "c1": time_fp32(fa, torch, 1, 256, 1, 64, False, 50),
            "large": time_fp32(fa, torch, 1, 4096, 16, 128, False, 10),
        }
        result["fp32"]["c1"]["note"] = "config 1: correctness case, latency-bound (4 workgroups)"
        log("bench: forward + backward with dropout")
        result["dropout"] = time_dropout(fa, torch, 2, 8192, 16, 64, 0.1, 10)
        log("bench: single-pass backward (atomic dQ) beside the two-pass backward")
        result["backward_single_pass"] = time_single_pass(fa, torch, 2, 8192, 16, 64, 20)
        log("bench: split-key decode against a long K/V cache")
        result["decode"] = {
            "nq1": time_decode(fa, torch, 8, 1, 32768, 32, 128, 6, 20),
            "nq4": time_decode(fa, torch, 8, 4, 32768, 32, 128, 6, 20),
        }

    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline on one head")
        got = {"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}
        result["cpu_baseline"], result["sample_parity_max_abs_err"] = cpu_baseline(w, host, got)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
