"""The static check of asm-issued LDS reads (exact_io_aware_39_amd.asm_check).

Synthetic assembly fragments check that the scan flags a use of a read's
destination before a wait that retires it, counts later LDS reads when
deciding what an lgkmcnt(n) wait retires, and refuses to carry a pending read
across a branch; the built kernels' assembly (written by the build next to the
objects) must be clean.
"""
import glob
import os

import pytest

from exact_io_aware_39_amd import asm_check

HEAD = "_Zkernel:\n"


def asm_read(text):
    return f";;#ASMSTART\n\t{text}\n;;#ASMEND\n"


def run(body):
    return asm_check.check_text(HEAD + body)


def test_use_after_full_wait_is_clean():
    probs, n = run(asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
                   + asm_read("s_waitcnt lgkmcnt(0)")
                   + "\tv_mfma_f32_32x32x16_bf16 v[20:35], v[10:13], v[40:43], v[20:35]\n")
    assert n == 1 and probs == []


def test_use_before_wait_is_flagged():
    probs, _ = run(asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
                   + "\tv_mfma_f32_32x32x16_bf16 v[20:35], v[10:13], v[40:43], v[20:35]\n"
                   + asm_read("s_waitcnt lgkmcnt(0)"))
    assert len(probs) == 1 and "before a wait retires it" in probs[0]


def test_overwrite_before_wait_is_flagged():
    probs, _ = run(asm_read("ds_read_b128 v[12:15], v3 offset:64")
                   + "\tv_mov_b32_e32 v13, 0\n")
    assert len(probs) == 1


def test_partial_wait_counts_later_reads():
    body = (asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
            + asm_read("ds_read_b64_tr_b16 v[12:13], v2 offset:512")
            + asm_read("s_waitcnt lgkmcnt(1)"))
    probs, _ = run(body + "\tv_add_u32_e32 v50, v10, v11\n" + asm_read("s_waitcnt lgkmcnt(0)"))
    assert probs == []                                   # first read retired by lgkmcnt(1)
    probs, _ = run(body + "\tv_add_u32_e32 v50, v12, v13\n" + asm_read("s_waitcnt lgkmcnt(0)"))
    assert len(probs) == 1                               # second one is not


def test_compiler_lds_ops_count_as_later():
    probs, _ = run(asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
                   + "\tds_read_b128 v[20:23], v4\n"
                   + "\ts_waitcnt lgkmcnt(1)\n"
                   + "\tv_add_u32_e32 v50, v10, v11\n")
    assert probs == []


def test_pending_read_across_branch_is_flagged():
    probs, _ = run(asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
                   + "\ts_cbranch_scc1 .LBB0_3\n")
    assert len(probs) == 1 and "branch" in probs[0]


def test_unrelated_registers_are_free():
    probs, _ = run(asm_read("ds_read_b64_tr_b16 v[10:11], v2 offset:0")
                   + "\tv_fma_f32 v30, v31, s4, -v32\n\tv_exp_f32_e32 v33, v30\n"
                   + asm_read("s_waitcnt lgkmcnt(0)"))
    assert probs == []


def test_built_kernels_are_clean():
    asms = glob.glob(os.path.join(os.path.dirname(asm_check.__file__), "_build", "*.hip.s"))
    if not asms:
        pytest.skip("library not built")
    total = 0
    for a in asms:
        probs, n = asm_check.check_file(a)
        assert probs == [], probs[:5]
        total += n
    assert total > 0
