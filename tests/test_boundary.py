"""The C ABI on the host: exported symbols and argument validation (no GPU).

Every call below is rejected by the library's host-side checks, which run
before any HIP call, so nothing is launched.  Pointer values are fake but
never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_io_aware_39_amd", "libfa.so")

OK, INVALID, UNSUPPORTED, LAUNCH, SCRATCH_LIMIT = 0, 1, 2, 3, 4
P = 0x10000          # a 16-byte aligned fake device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfa.so not built: run python -m exact_io_aware_39_amd.build")
    lib = ctypes.CDLL(LIB)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("fa_forward", "fa_forward_f32"):
        getattr(lib, name).argtypes = [vp] * 5 + [i] * 4 + [f, i, vp]
        getattr(lib, name).restype = i
    for name in ("fa_backward", "fa_backward_f32"):
        getattr(lib, name).argtypes = [vp] * 10 + [i] * 4 + [f, i, vp]
        getattr(lib, name).restype = i
    lib.fa_backward_preprocess.argtypes = [vp] * 4 + [i] * 4 + [vp]
    lib.fa_backward_preprocess.restype = i
    lib.fa_backward_dqdkdv.argtypes = [vp] * 8 + [i] * 4 + [f, i, vp]
    lib.fa_backward_dqdkdv.restype = i
    lib.fa_backward_dkdv.argtypes = [vp] * 7 + [i] * 4 + [f, i, vp]
    lib.fa_backward_dkdv.restype = i
    lib.fa_backward_dq.argtypes = [vp] * 6 + [i] * 4 + [f, i, vp]
    lib.fa_backward_dq.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i] * 4
    lib.fa_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_forward_cross.argtypes = [vp] * 5 + [i] * 5 + [f, i, vp]
    lib.fa_forward_cross.restype = i
    lib.fa_backward_cross.argtypes = [vp] * 10 + [i] * 5 + [f, i, vp]
    lib.fa_backward_cross.restype = i
    lib.fa_decode.argtypes = [vp] * 6 + [i] * 5 + [f, i, i, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_splits.argtypes = [i] * 5
    lib.fa_decode_splits.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i] * 6
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_backward_noalloc.argtypes = [vp] * 9 + [i] * 4 + [f, i, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_single_pass.argtypes = [vp] * 10 + [i] * 4 + [f, i, vp]
    lib.fa_backward_single_pass.restype = i
    lib.fa_backward_single_pass_workspace_bytes.argtypes = [i] * 4
    lib.fa_backward_single_pass_workspace_bytes.restype = ctypes.c_size_t
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_forward_dropout.argtypes = [vp] * 5 + [i] * 4 + [f, i, f, u64, u32, vp]
    lib.fa_forward_dropout.restype = i
    lib.fa_backward_dropout.argtypes = [vp] * 10 + [i] * 4 + [f, i, f, u64, u32, vp]
    lib.fa_backward_dropout.restype = i
    lib.fa_forward_fp8.argtypes = [vp] * 3 + [f] * 3 + [vp] * 3 + [i] * 5 + [f, i, vp]
    lib.fa_forward_fp8.restype = i
    lib.fa_forward_fp8_workspace_bytes.argtypes = [i] * 4
    lib.fa_forward_fp8_workspace_bytes.restype = ctypes.c_size_t
    return lib


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "fa_forward", "fa_forward_f32", "fa_backward", "fa_backward_f32",
        "fa_backward_preprocess", "fa_backward_dqdkdv", "fa_backward_dkdv", "fa_backward_dq",
        "fa_backward_workspace_bytes", "fa_status_string",
        "fa_decode", "fa_decode_splits", "fa_decode_workspace_bytes", "fa_forward_cross",
        "fa_backward_cross", "fa_forward_fp8", "fa_forward_fp8_workspace_bytes",
        "fa_forward_dropout", "fa_backward_dropout",
        "fa_backward_single_pass", "fa_backward_single_pass_workspace_bytes",
        "fa_backward_noalloc"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_sync_check_build_exports_the_same_abi():
    """libfa_synccheck.so (the race-detection build) exports every declared
    entry point too, and its host checks agree with libfa.so's."""
    path = os.path.join(ROOT, "exact_io_aware_39_amd", "libfa_synccheck.so")
    if not os.path.exists(path):
        pytest.fail("libfa_synccheck.so not built: run python -m exact_io_aware_39_amd.build")
    sc = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(sc, name), name
    sc.fa_backward_workspace_bytes.argtypes = [ctypes.c_int] * 4
    sc.fa_backward_workspace_bytes.restype = ctypes.c_size_t
    sc.fa_status_string.argtypes = [ctypes.c_int]
    sc.fa_status_string.restype = ctypes.c_char_p
    normal = ctypes.CDLL(LIB)
    normal.fa_backward_workspace_bytes.argtypes = [ctypes.c_int] * 4
    normal.fa_backward_workspace_bytes.restype = ctypes.c_size_t
    for shape in ((1, 1, 1, 64), (2, 3, 300, 128), (1, 2, 600, 256)):
        assert sc.fa_backward_workspace_bytes(*shape) == normal.fa_backward_workspace_bytes(*shape)
    assert sc.fa_status_string(4).startswith(b"FA_ERR_SCRATCH_LIMIT")


def _fwd(lib, name="fa_forward", ptrs=(P, P, P, P, P), B=1, H=1, N=128, d=64, scale=0.125, causal=0):
    return getattr(lib, name)(*ptrs, B, H, N, d, scale, causal, None)


def _bwd(lib, name="fa_backward", ptrs=(P,) * 10, B=1, H=1, N=128, d=64, scale=0.125, causal=0):
    return getattr(lib, name)(*ptrs, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("name", ["fa_forward", "fa_forward_f32"])
def test_forward_rejects_bad_arguments(lib, name):
    for d in (0, 32, 96, 512) + ((256,) if name == "fa_forward_f32" else ()):
        assert _fwd(lib, name, d=d) == UNSUPPORTED
    if name == "fa_forward":
        # d = 256 passes the head-size check (a null pointer is the first error)
        assert _fwd(lib, name, d=256, ptrs=(None,) + (P,) * 4) == INVALID
    for B, H, N in ((0, 1, 8), (1, 0, 8), (1, 1, 0), (-1, 1, 8)):
        assert _fwd(lib, name, B=B, H=H, N=N) == INVALID
    assert _fwd(lib, name, N=(1 << 20) + 1) == UNSUPPORTED
    assert _fwd(lib, name, B=1 << 11, H=1 << 10) == UNSUPPORTED
    assert _fwd(lib, name, H=(1 << 17) + 1, d=128) == UNSUPPORTED
    for s in (float("nan"), float("inf"), float("-inf")):
        assert _fwd(lib, name, scale=s) == INVALID
    assert _fwd(lib, name, scale=-0.5) == UNSUPPORTED
    assert _fwd(lib, name, causal=2) == INVALID
    assert _fwd(lib, name, causal=-1) == INVALID
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = None
        assert _fwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    for i in range(4):                       # tensors need 16-byte alignment
        ptrs = [P] * 5
        ptrs[i] = P + 8
        assert _fwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    assert _fwd(lib, name, ptrs=(P, P, P, P, P + 2)) == INVALID   # LSE needs 4-byte alignment


@pytest.mark.parametrize("name", ["fa_backward", "fa_backward_f32"])
def test_backward_rejects_bad_arguments(lib, name):
    assert _bwd(lib, name, d=80) == UNSUPPORTED
    if name == "fa_backward":
        assert _bwd(lib, name, d=256, ptrs=(None,) + (P,) * 9) == INVALID
    else:
        assert _bwd(lib, name, d=256) == UNSUPPORTED
    assert _bwd(lib, name, N=0) == INVALID
    assert _bwd(lib, name, scale=float("nan")) == INVALID
    assert _bwd(lib, name, causal=3) == INVALID
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    for i in (0, 1, 2, 3, 4, 6, 7, 8):         # Q K V O dO dQ dK dV: 16-byte alignment
        ptrs = [P] * 10
        ptrs[i] = P + 4
        assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    for i in (5, 9):                          # LSE and workspace: 4-byte alignment
        ptrs = [P] * 10
        ptrs[i] = P + 2
        assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID


def test_single_pass_rejects_bad_arguments(lib):
    name = "fa_backward_single_pass"
    assert _bwd(lib, name, d=80) == UNSUPPORTED
    assert _bwd(lib, name, d=256) == UNSUPPORTED      # d = 64 and 128 only
    assert _bwd(lib, name, N=0) == INVALID
    assert _bwd(lib, name, B=-1) == INVALID
    assert _bwd(lib, name, scale=float("inf")) == INVALID
    assert _bwd(lib, name, causal=2) == INVALID
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    for i in (0, 1, 2, 3, 4, 6, 7, 8, 9):      # tensors and the workspace: 16-byte alignment
        ptrs = [P] * 10
        ptrs[i] = P + 4
        assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID
    ptrs = [P] * 10
    ptrs[5] = P + 2                             # LSE: 4-byte alignment
    assert _bwd(lib, name, ptrs=tuple(ptrs)) == INVALID


def test_noalloc_rejects_bad_arguments(lib):
    """The allocation-free backward: fa_backward's checks, and the size of its
    static scratch (2^21 query rows), all before any HIP call."""
    def call(ptrs=(P,) * 9, B=1, H=1, N=128, d=64, scale=0.125, causal=0):
        return lib.fa_backward_noalloc(*ptrs, B, H, N, d, scale, causal, None)
    assert call(d=80) == UNSUPPORTED
    assert call(N=0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(causal=2) == INVALID
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert call(ptrs=tuple(ptrs)) == INVALID
    assert call(ptrs=(P,) * 5 + (P + 2,) + (P,) * 3) == INVALID       # LSE 4-byte alignment
    assert call(ptrs=(P + 4,) + (P,) * 8) == INVALID                  # Q 16-byte alignment
    assert call(B=1, H=32, N=65537) == SCRATCH_LIMIT
    assert call(B=4, H=16, N=32769) == SCRATCH_LIMIT
    assert call(B=2, H=16, N=65537, d=256) == SCRATCH_LIMIT


def test_single_pass_workspace_bytes(lib):
    f = lib.fa_backward_single_pass_workspace_bytes
    # [-D | -LSE log2 e | padding to 16 bytes | B N H d floats]
    assert f(2, 16, 8192, 64) == (2 * 2 * 16 * 8192 + 2 * 8192 * 16 * 64) * 4
    assert f(1, 1, 1, 64) == (4 + 64) * 4
    assert f(1, 3, 5, 128) == (32 + 3 * 5 * 128) * 4
    assert f(1, 1, 1, 256) == 0
    assert f(0, 1, 1, 64) == 0


def test_backward_passes_reject_bad_arguments(lib):
    assert lib.fa_backward_preprocess(P, P, P, P, 1, 1, 128, 96, None) == UNSUPPORTED
    assert lib.fa_backward_preprocess(P, P, P, P, 1, 0, 128, 64, None) == INVALID
    for i in range(4):
        ptrs = [P] * 4
        ptrs[i] = None
        assert lib.fa_backward_preprocess(*ptrs, 1, 1, 128, 64, None) == INVALID
    assert lib.fa_backward_preprocess(P + 8, P, P, P, 1, 1, 128, 64, None) == INVALID
    assert lib.fa_backward_preprocess(P, P + 8, P, P, 1, 1, 128, 64, None) == INVALID
    assert lib.fa_backward_preprocess(P, P, P + 2, P, 1, 1, 128, 64, None) == INVALID
    assert lib.fa_backward_preprocess(P, P, P, P + 2, 1, 1, 128, 64, None) == INVALID
    for name, n, stats in (("fa_backward_dqdkdv", 8, (4,)), ("fa_backward_dkdv", 7, (4,)),
                           ("fa_backward_dq", 6, (4,))):
        fn = getattr(lib, name)
        assert fn(*([P] * n), 1, 1, 128, 32, 0.1, 0, None) == UNSUPPORTED
        assert fn(*([P] * n), 1, 1, 128, 64, float("nan"), 0, None) == INVALID
        assert fn(*([P] * n), 1, 1, 128, 64, 0.1, 5, None) == INVALID
        for i in range(n):
            ptrs = [P] * n
            ptrs[i] = None
            assert fn(*ptrs, 1, 1, 128, 64, 0.1, 1, None) == INVALID
        for i in range(n):                  # workspace (5th) needs 4-byte, tensors 16-byte alignment
            ptrs = [P] * n
            ptrs[i] = P + (2 if i in stats else 8)
            assert fn(*ptrs, 1, 1, 128, 64, 0.1, 1, None) == INVALID


def test_head_size_256_only_on_the_bf16_forward_and_backward(lib):
    assert lib.fa_backward_workspace_bytes(1, 2, 100, 256) == 8 * 2 * 100
    assert lib.fa_decode_workspace_bytes(1, 2, 1, 100, 256, 0) == 0
    assert lib.fa_forward_fp8_workspace_bytes(1, 2, 100, 256) == 0
    assert lib.fa_forward_cross(None, P, P, P, P, 1, 2, 10, 20, 256, 0.1, 1, None) == INVALID
    assert lib.fa_backward_cross(None, *([P] * 9), 1, 2, 10, 20, 256, 0.1, 1, None) == INVALID
    for name in ("fa_backward_dqdkdv", "fa_backward_dkdv", "fa_backward_dq"):
        n = {"fa_backward_dqdkdv": 8, "fa_backward_dkdv": 7, "fa_backward_dq": 6}[name]
        assert getattr(lib, name)(None, *([P] * (n - 1)), 1, 2, 100, 256, 0.1, 1, None) == INVALID
    assert lib.fa_backward_preprocess(None, P, P, P, 1, 2, 100, 256, None) == INVALID
    assert lib.fa_decode(*([P] * 6), 1, 2, 1, 100, 256, 0.1, 1, 0, None) == UNSUPPORTED
    assert lib.fa_forward_fp8(P, P, P, 1.0, 1.0, 1.0, P, P, P, 1, 2, 10, 20, 256, 0.1, 1, None) == UNSUPPORTED


def test_workspace_bytes(lib):
    assert lib.fa_backward_workspace_bytes(2, 16, 8192, 64) == 2 * 2 * 16 * 8192 * 4
    assert lib.fa_backward_workspace_bytes(1, 1, 1, 128) == 8
    assert lib.fa_backward_workspace_bytes(0, 16, 8192, 64) == 0
    assert lib.fa_backward_workspace_bytes(2, 16, 8192, 96) == 0


def test_forward_cross_rejects_bad_arguments(lib):
    def call(B=1, H=2, Nq=100, Nk=300, d=64, scale=0.1, causal=1, ptrs=(P,) * 5):
        return lib.fa_forward_cross(*ptrs, B, H, Nq, Nk, d, scale, causal, None)
    assert call(d=96) == UNSUPPORTED
    assert call(Nq=0) == INVALID
    assert call(Nk=0) == INVALID
    assert call(Nq=301, causal=1) == INVALID        # more rows than keys under the mask
    assert call(Nk=(1 << 20) + 1) == UNSUPPORTED
    assert call(Nq=(1 << 20) + 1, causal=0) == UNSUPPORTED
    assert call(scale=float("nan")) == INVALID
    assert call(causal=7) == INVALID
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = None
        assert call(ptrs=tuple(ptrs)) == INVALID
        ptrs[i] = P + (2 if i == 4 else 8)
        assert call(ptrs=tuple(ptrs)) == INVALID


def test_forward_fp8_rejects_bad_arguments(lib):
    def call(B=1, H=2, Nq=100, Nk=300, d=64, scale=0.1, causal=1, ds=(0.5, 0.5, 0.5), ptrs=(P,) * 6):
        q, k, v, o, lse, ws = ptrs
        return lib.fa_forward_fp8(q, k, v, *ds, o, lse, ws, B, H, Nq, Nk, d, scale, causal, None)
    assert call(d=96) == UNSUPPORTED
    assert call(Nq=0) == INVALID
    assert call(Nk=0) == INVALID
    assert call(Nq=301, causal=1) == INVALID
    assert call(Nk=(1 << 20) + 1) == UNSUPPORTED
    assert call(scale=float("inf")) == INVALID
    assert call(causal=2) == INVALID
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        for j in range(3):
            ds = [0.5, 0.5, 0.5]
            ds[j] = bad
            assert call(ds=tuple(ds)) == INVALID, (j, bad)
    assert call(scale=3e38, ds=(1e10, 1e10, 1.0)) == INVALID    # scale * dq * dk overflows
    for j in range(6):
        ptrs = [P] * 6
        ptrs[j] = None
        assert call(ptrs=tuple(ptrs)) == INVALID
        ptrs[j] = P + (2 if j == 4 else 8)
        assert call(ptrs=tuple(ptrs)) == INVALID


def test_dropout_rejects_bad_arguments(lib):
    def fwd(p=0.1, d=64, N=100, causal=1, ptrs=(P,) * 5):
        return lib.fa_forward_dropout(*ptrs, 1, 2, N, d, 0.125, causal, p, 12345, 0, None)

    def bwd(p=0.1, d=64, N=100, causal=1, ptrs=(P,) * 10):
        return lib.fa_backward_dropout(*ptrs, 1, 2, N, d, 0.125, causal, p, 12345, 0, None)
    for call in (fwd, bwd):
        for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
            assert call(p=p) == INVALID, p
        assert call(d=96) == UNSUPPORTED
        assert call(N=0) == INVALID
        assert call(causal=2) == INVALID
    for j in range(5):
        ptrs = [P] * 5
        ptrs[j] = None
        assert fwd(ptrs=tuple(ptrs)) == INVALID
    for j in range(10):
        ptrs = [P] * 10
        ptrs[j] = None
        assert bwd(ptrs=tuple(ptrs)) == INVALID
    # p = 0 and d = 256 pass the checks (a null pointer is then the first error)
    assert fwd(p=0.0, d=256, ptrs=(None,) + (P,) * 4) == INVALID
    assert bwd(p=0.0, d=256, ptrs=(None,) + (P,) * 9) == INVALID


def test_forward_fp8_workspace_bytes(lib):
    assert lib.fa_forward_fp8_workspace_bytes(4, 16, 4096, 128) == 4 * 16 * 128 * 4096
    assert lib.fa_forward_fp8_workspace_bytes(1, 2, 65, 64) == 2 * 64 * 128
    assert lib.fa_forward_fp8_workspace_bytes(1, 1, 1, 64) == 64 * 64
    assert lib.fa_forward_fp8_workspace_bytes(1, 1, 0, 64) == 0
    assert lib.fa_forward_fp8_workspace_bytes(1, 1, 64, 96) == 0


def test_backward_cross_rejects_bad_arguments(lib):
    def call(B=1, H=2, Nq=100, Nk=300, d=64, scale=0.1, causal=1, ptrs=(P,) * 10):
        return lib.fa_backward_cross(*ptrs, B, H, Nq, Nk, d, scale, causal, None)
    assert call(d=96) == UNSUPPORTED
    assert call(Nq=0) == INVALID
    assert call(Nk=0) == INVALID
    assert call(Nq=301, causal=1) == INVALID        # more rows than keys under the mask
    assert call(Nk=(1 << 20) + 1) == UNSUPPORTED
    assert call(Nq=(1 << 20) + 1, causal=0) == UNSUPPORTED
    assert call(scale=float("nan")) == INVALID
    assert call(scale=-0.5) == UNSUPPORTED
    assert call(causal=3) == INVALID
    stats = (5, 9)                                   # LSE and workspace: 4-byte alignment
    for i in range(10):
        ptrs = [P] * 10
        ptrs[i] = None
        assert call(ptrs=tuple(ptrs)) == INVALID
        ptrs[i] = P + (2 if i in stats else 8)
        assert call(ptrs=tuple(ptrs)) == INVALID


def _dec(lib, B=1, H=2, Nq=1, Nk=100, d=64, scale=0.1, causal=1, splits=0, ptrs=(P,) * 6):
    return lib.fa_decode(*ptrs, B, H, Nq, Nk, d, scale, causal, splits, None)


def test_decode_rejects_bad_arguments(lib):
    assert _dec(lib, d=96) == UNSUPPORTED
    assert _dec(lib, Nq=0) == INVALID
    assert _dec(lib, Nq=33) == UNSUPPORTED
    assert _dec(lib, Nq=5, Nk=4, causal=1) == INVALID       # more rows than keys under the mask
    assert _dec(lib, splits=-1) == INVALID
    assert _dec(lib, splits=4097) == UNSUPPORTED
    assert _dec(lib, Nk=0) == INVALID
    assert _dec(lib, Nk=(1 << 20) + 1) == UNSUPPORTED
    assert _dec(lib, scale=float("inf")) == INVALID
    assert _dec(lib, scale=-1.0) == UNSUPPORTED
    assert _dec(lib, causal=2) == INVALID
    for i in range(6):
        ptrs = [P] * 6
        ptrs[i] = None
        assert _dec(lib, ptrs=tuple(ptrs)) == INVALID
    for i in range(6):                       # Q K V O: 16-byte alignment; LSE, workspace: 4-byte
        ptrs = [P] * 6
        ptrs[i] = P + (2 if i >= 4 else 8)
        assert _dec(lib, ptrs=tuple(ptrs)) == INVALID


def test_decode_splits_and_workspace(lib):
    # about 1024 workgroups in all, at least 8 blocks of 32 keys a chunk
    assert lib.fa_decode_splits(8, 32, 1, 16384, 128) == 4
    assert lib.fa_decode_splits(1, 1, 1, 31, 64) == 1
    assert lib.fa_decode_splits(1, 1, 4, 1 << 20, 64) == 1024
    assert lib.fa_decode_splits(1, 1, 33, 100, 64) == 0
    assert lib.fa_decode_workspace_bytes(8, 32, 1, 16384, 128, 0) == 8 * 32 * 4 * 1 * 129 * 4
    assert lib.fa_decode_workspace_bytes(2, 3, 5, 1000, 64, 7) == 2 * 3 * 7 * 5 * 65 * 4
    assert lib.fa_decode_workspace_bytes(2, 3, 5, 1000, 64, 4097) == 0
    assert lib.fa_decode_workspace_bytes(2, 3, 0, 1000, 64, 1) == 0


def test_status_strings(lib):
    for code, key in ((OK, b"FA_OK"), (INVALID, b"FA_ERR_INVALID_ARG"),
                      (UNSUPPORTED, b"FA_ERR_UNSUPPORTED"), (LAUNCH, b"FA_ERR_LAUNCH"),
                      (SCRATCH_LIMIT, b"FA_ERR_SCRATCH_LIMIT")):
        assert lib.fa_status_string(code).startswith(key)
    assert b"unknown" in lib.fa_status_string(99)


def test_python_binding_reports_status_names():
    from exact_io_aware_39_amd import fa_status_string, FaError
    assert fa_status_string(2).startswith("FA_ERR_UNSUPPORTED")
    assert "FA_ERR_INVALID_ARG" in str(FaError(1, "fa_forward"))


def _bnhd(B=2, N=64, H=3, d=64, dtype=None):
    import torch
    return torch.zeros((B, N, H, d), dtype=dtype or torch.bfloat16)


def _wrapper_calls():
    """(name, call with every shape right, {tensor: wrong-shaped replacement})."""
    import torch
    import exact_io_aware_39_amd._lib as L
    B, N, H, d = 2, 64, 3, 64
    t = lambda: _bnhd(B, N, H, d)                                  # noqa: E731
    lse = lambda: torch.zeros((B, H, N), dtype=torch.float32)       # noqa: E731
    ws = lambda: torch.zeros(2 * B * H * N, dtype=torch.float32)    # noqa: E731
    short, bad_lse = _bnhd(B, N - 8, H, d), torch.zeros((B, H, N - 8), dtype=torch.float32)
    calls = [
        ("fa_forward", lambda a: L.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, True),
         ["k", "v", "o", "lse"]),
        ("fa_backward", lambda a: L.fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                               a["dk"], a["dv"], a["ws"], 0.1, True),
         ["k", "v", "o", "do", "dq", "dk", "dv", "lse"]),
        ("fa_backward_single_pass", lambda a: L.fa_backward_single_pass(
            a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"], 0.1, True),
         ["k", "v", "o", "do", "dq", "dk", "dv", "lse"]),
        ("fa_backward_preprocess", lambda a: L.fa_backward_preprocess(a["o"], a["do"], a["lse"], a["ws"]),
         ["do", "lse"]),
        ("fa_backward_dqdkdv", lambda a: L.fa_backward_dqdkdv(a["q"], a["k"], a["v"], a["do"], a["ws"], a["dq"],
                                                             a["dk"], a["dv"], 0.1, True),
         ["k", "v", "do", "dq", "dk", "dv"]),
        ("fa_backward_dkdv", lambda a: L.fa_backward_dkdv(a["q"], a["k"], a["v"], a["do"], a["ws"], a["dk"],
                                                         a["dv"], 0.1, True),
         ["k", "v", "do", "dk", "dv"]),
        ("fa_backward_dq", lambda a: L.fa_backward_dq(a["q"], a["k"], a["v"], a["do"], a["ws"], a["dq"], 0.1, True),
         ["k", "v", "do", "dq"]),
        ("fa_forward_dropout", lambda a: L.fa_forward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, True,
                                                             0.1, 1),
         ["k", "v", "o", "lse"]),
        ("fa_backward_dropout", lambda a: L.fa_backward_dropout(
            a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"], 0.1, True, 0.1, 1),
         ["k", "v", "o", "do", "dq", "dk", "dv", "lse"]),
        ("fa_forward_cross", lambda a: L.fa_forward_cross(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, False),
         ["o", "lse"]),
        ("fa_backward_cross", lambda a: L.fa_backward_cross(
            a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"], 0.1, False),
         ["o", "do", "dq", "dk", "dv", "lse"]),
        ("fa_decode", lambda a: L.fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], 0.1, False),
         ["o", "lse"]),
    ]
    for name, call, wrong in calls:
        def make(name=name):
            return {"q": t(), "k": t(), "v": t(), "o": t(), "do": t(), "dq": t(), "dk": t(), "dv": t(),
                    "lse": lse(), "ws": ws()}
        yield name, call, make, wrong, short, bad_lse


@pytest.mark.parametrize("case", list(_wrapper_calls()), ids=lambda c: c[0])
def test_binding_rejects_mismatched_shapes(case):
    """Each wrapper checks every tensor's shape against q's (lse against
    [B, H, N]) before it touches the library, so a short K or a small LSE is
    a ValueError, not an out-of-bounds device access.  The tensors here are on
    the CPU: with the shapes right the call gets as far as the device check."""
    name, call, make, wrong, short, bad_lse = case
    with pytest.raises(ValueError, match="CUDA"):
        call(make())
    for which in wrong:
        args = make()
        args[which] = bad_lse if which == "lse" else short
        with pytest.raises(ValueError, match="shape|must share"):
            call(args)
