"""Static check of the asm-issued LDS reads in the generated gfx950 assembly.

The kernels issue some LDS reads from inline asm (see ``fa_common.hpp``), which
hides them from the compiler's wait-count bookkeeping.  Their results are only
valid once an ``s_waitcnt lgkmcnt(n)`` has retired them: LDS operations
complete in issue order, so such a wait retires every LDS read that has at
least n LDS operations issued after it.  This module scans the assembly of
every kernel and reports any instruction that reads or writes a destination
register of an asm-issued read before a wait retires it, and any branch or
block boundary crossed while such a read is pending.

    python -m exact_io_aware_39_amd.asm_check file.s [...]
"""
from __future__ import annotations

import re
import sys

_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
_LABEL = re.compile(r"^\.LBB\d+_\d+:")


def _regs(text: str) -> set:
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def check_text(text: str, name: str = "<asm>"):
    """Returns (problems, number of asm-issued LDS reads seen)."""
    problems = []
    kernel = None
    pending = []     # [destination registers, LDS operations issued after it]
    in_asm = False
    n_reads = 0

    def flush(where, why):
        if pending:
            problems.append(f"{name}:{where}: {kernel}: {why} with {len(pending)} asm LDS read(s) pending")
        pending.clear()

    for no, raw in enumerate(text.split("\n"), 1):
        stripped = raw.strip()
        if stripped == ";;#ASMSTART":
            in_asm = True
            continue
        if stripped == ";;#ASMEND":
            in_asm = False
            continue
        code = raw.split(";")[0].rstrip()
        if code.startswith("_Z") and code.endswith(":"):
            kernel = code[:-1]
            pending.clear()
            continue
        s = code.strip()
        if not s:
            continue
        if _LABEL.match(s):
            flush(no, "block boundary")
            continue
        if s.startswith("."):
            continue
        op = s.split()[0]
        if op.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                k = int(m.group(1))
                pending[:] = [p for p in pending if p[1] < k]
            continue
        operands = s[len(op):]
        used = _regs(operands)
        is_ds = op.startswith("ds_")
        if in_asm and op.startswith("ds_read"):
            dest = _regs(operands.split(",")[0])
            for p in pending:
                if p[0] & used:
                    problems.append(f"{name}:{no}: {kernel}: '{s}' touches a pending asm LDS read")
                p[1] += 1
            pending.append([dest, 0])
            n_reads += 1
            continue
        for p in pending:
            if p[0] & used:
                problems.append(f"{name}:{no}: {kernel}: '{s}' touches v{sorted(p[0])} before a wait retires it")
        if is_ds:
            for p in pending:
                p[1] += 1
        if op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
            flush(no, "branch")
    return problems, n_reads


def check_file(path: str):
    with open(path) as f:
        return check_text(f.read(), path)


if __name__ == "__main__":
    bad = 0
    for p in sys.argv[1:]:
        probs, n = check_file(p)
        print(f"{p}: {n} asm LDS reads, {len(probs)} problems")
        for line in probs[:20]:
            print("  ", line)
        bad += len(probs)
    sys.exit(1 if bad else 0)
