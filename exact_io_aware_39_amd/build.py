"""Build libfa.so (the gfx950 kernels and the C ABI) in place with hipcc.

    python -m exact_io_aware_39_amd.build [-v]

Every source under csrc/ is compiled for gfx950 only.  Packed-fp32 VALU
instructions are disabled (-packed-fp32-ops): the kernels are written in
scalar fp32 for the softmax arithmetic.

The same sources are also built with -DFA_SYNC_CHECK into
libfa_synccheck.so, the race-detection build: every asm-issued LDS read and
every global -> LDS copy completes at once and every workgroup barrier drains
all memory operations first (csrc/fa_common.hpp).  It exports the same C ABI
and must give bit-identical results; tests/test_gpu_sync_check.py compares
the two.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
OUT_SYNC_CHECK = os.path.join(PKG, "libfa_synccheck.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Extra flags per source.  The d = 128 backward kernels run at one wave per
# SIMD; at that budget the compiler otherwise gives every MFMA the AGPR form
# and moves the score results, which the vector unit reads, out of AGPRs (on
# MI355X the d = 128 backward measured 18-20% faster causal, 7% without a
# mask, with this flag; bitwise the same results; the d = 64 kernels, which
# fit in VGPRs, are unaffected).
FILE_FLAGS = {
    "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return exe


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, obj, verbose, extra=()):
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def _device_asm(src, out, verbose):
    """gfx950 assembly of one kernel source (what the object file contains)."""
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "--cuda-device-only", "-S",
           src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {os.path.basename(src)}:\n{r.stderr}")
    return out


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, sync_check: bool = True) -> str:
    """Compile every source, check the asm-issued LDS reads in the generated
    assembly, and link libfa.so next to this file (and, with `sync_check`,
    the sync-check build libfa_synccheck.so); returns the path of libfa.so."""
    from . import asm_check
    objdir = os.path.join(PKG, "_build")
    syncdir = os.path.join(PKG, "_build", "sync_check")
    os.makedirs(syncdir, exist_ok=True)
    srcs = _sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    sync_objs = [os.path.join(syncdir, os.path.basename(s) + ".o") for s in srcs]
    hips = [s for s in srcs if s.endswith(".hip")]
    asms = [os.path.join(objdir, os.path.basename(s) + ".s") for s in hips]
    jobs = [(_compile, so, ob, ()) for so, ob in zip(srcs, objs)]
    jobs += [(_device_asm, so, a, None) for so, a in zip(hips, asms)]
    if sync_check:
        jobs += [(_compile, so, ob, ("-DFA_SYNC_CHECK",)) for so, ob in zip(srcs, sync_objs)]
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))

    def run(j):
        f, src, out, extra = j
        return f(src, out, verbose) if extra is None else f(src, out, verbose, extra)

    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, jobs))
    problems = []
    for a in asms:
        problems += asm_check.check_file(a)[0]
    if problems:
        raise RuntimeError("asm-issued LDS reads used before their wait:\n" + "\n".join(problems[:20]))
    _link(objs, OUT, verbose)
    if sync_check:
        _link(sync_objs, OUT_SYNC_CHECK, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
