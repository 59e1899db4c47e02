"""Build libfa.so (the gfx950 kernels and the C ABI) in place with hipcc.

    python -m exact_io_aware_39_amd.build [-v]

Every source under csrc/ is compiled for gfx950 only.  Packed-fp32 VALU
instructions are disabled (-packed-fp32-ops): the kernels are written in
scalar fp32 for the softmax arithmetic.
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


def _compile(src, obj, verbose):
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
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


def build(verbose: bool = False) -> str:
    """Compile every source, check the asm-issued LDS reads in the generated
    assembly, and link libfa.so next to this file; returns its path."""
    from . import asm_check

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = _sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    hips = [s for s in srcs if s.endswith(".hip")]
    asms = [os.path.join(objdir, os.path.basename(s) + ".s") for s in hips]
    jobs = [(_compile, so, ob) for so, ob in zip(srcs, objs)] + [(_device_asm, so, a) for so, a in zip(hips, asms)]
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: j[0](j[1], j[2], verbose), jobs))
    problems = []
    for a in asms:
        problems += asm_check.check_file(a)[0]
    if problems:
        raise RuntimeError("asm-issued LDS reads used before their wait:\n" + "\n".join(problems[:20]))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
