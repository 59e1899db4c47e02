"""ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: each function here turns torch tensors into device
pointers and sizes and calls the C entry point of the same name on the current
torch stream.  Nothing is computed in Python and there is no fallback: if the
library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
# The race-detection build of the same sources and C ABI (-DFA_SYNC_CHECK):
# every LDS read and global -> LDS copy completes at once, every barrier
# drains all memory operations first; results must equal libfa.so's bit for bit.
SYNC_CHECK_LIB_PATH = os.path.join(_HERE, "libfa_synccheck.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH, FA_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4

_libs = {}            # path -> loaded CDLL
_active = None        # path the wrappers call; None = LIB_PATH


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the library the wrappers call (libfa.so unless use_library()
    says otherwise), or the one at `path`, once; raise if it is not built."""
    path = path or _active or LIB_PATH
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_io_aware_39_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd_args = [P, P, P, P, P, I, I, I, I, F, I, P]
    bwd_args = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    for name, args in (("fa_forward", fwd_args), ("fa_forward_f32", fwd_args),
                       ("fa_backward", bwd_args), ("fa_backward_f32", bwd_args)):
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, I
    lib.fa_backward_noalloc.argtypes = [P] * 9 + [I, I, I, I, F, I, P]
    lib.fa_backward_noalloc.restype = I
    lib.fa_backward_preprocess.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.fa_backward_preprocess.restype = I
    for name, nptr in (("fa_backward_dqdkdv", 8), ("fa_backward_dkdv", 7), ("fa_backward_dq", 6)):
        fn = getattr(lib, name)
        fn.argtypes = [P] * nptr + [I, I, I, I, F, I, P]
        fn.restype = I
    lib.fa_backward_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_backward_single_pass.argtypes = bwd_args
    lib.fa_backward_single_pass.restype = I
    lib.fa_backward_single_pass_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_backward_single_pass_workspace_bytes.restype = S
    lib.fa_backward_workspace_bytes.restype = S
    lib.fa_forward_cross.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_forward_cross.restype = I
    lib.fa_backward_cross.argtypes = [P] * 10 + [I, I, I, I, I, F, I, P]
    lib.fa_backward_cross.restype = I
    lib.fa_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.fa_decode.restype = I
    lib.fa_decode_splits.argtypes = [I, I, I, I, I]
    lib.fa_decode_splits.restype = I
    lib.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.fa_decode_workspace_bytes.restype = S
    U64, U32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_forward_dropout.argtypes = [P] * 5 + [I] * 4 + [F, I, F, U64, U32, P]
    lib.fa_forward_dropout.restype = I
    lib.fa_backward_dropout.argtypes = [P] * 10 + [I] * 4 + [F, I, F, U64, U32, P]
    lib.fa_backward_dropout.restype = I
    lib.fa_forward_fp8.argtypes = [P, P, P, F, F, F, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_forward_fp8.restype = I
    lib.fa_forward_fp8_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_forward_fp8_workspace_bytes.restype = S
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    _libs[path] = lib
    return lib


@contextlib.contextmanager
def use_library(path: str):
    """Inside the block every wrapper calls the library at `path` (another
    build of the same C ABI, e.g. SYNC_CHECK_LIB_PATH) instead of libfa.so."""
    global _active
    load(path)
    prev, _active = _active, path
    try:
        yield
    finally:
        _active = prev


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_backward_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_backward_workspace_bytes(B, H, N, d))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(q):
    if q.dim() != 4:
        raise ValueError(f"expected a [B, N, H, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _check(ts, dtype):
    for t in ts:
        if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"expected contiguous {dtype} CUDA tensors, got {t.dtype} on {t.device}")
    devs = {t.device for t in ts}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


def _same_shape(where, ref, named):
    """Every tensor of `named` ({name: tensor}) must have the shape of `ref`."""
    want = tuple(ref.shape)
    for name, t in named.items():
        if tuple(t.shape) != want:
            raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {want}")


def _lse_shape(where, lse, B, H, N, name="lse"):
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"{where}: {name} has shape {tuple(lse.shape)}, expected [B, H, N] = {(B, H, N)}")


def _call(name, status):
    if status != FA_OK:
        raise FaError(status, name)


def fa_forward(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    """fa_forward / fa_forward_f32 on [B, N, H, d] tensors (bf16 or fp32)."""
    B, N, H, d = _shape(q)
    name = "fa_forward" if q.dtype == torch.bfloat16 else "fa_forward_f32"
    _same_shape(name, q, {"k": k, "v": v, "o": o})
    _lse_shape(name, lse, B, H, N)
    _check((q, k, v, o), q.dtype)
    _check((lse,), torch.float32)
    fn = getattr(load(), name)
    _call(name, fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                   int(bool(causal)), _stream(stream)))


def fa_backward(q, k, v, o, do, lse, dq, dk, dv, workspace, scale: float, causal: bool, stream=None):
    """fa_backward / fa_backward_f32 on [B, N, H, d] tensors (bf16 or fp32)."""
    B, N, H, d = _shape(q)
    name = "fa_backward" if q.dtype == torch.bfloat16 else "fa_backward_f32"
    _same_shape(name, q, {"k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv})
    _lse_shape(name, lse, B, H, N)
    _check((q, k, v, o, do, dq, dk, dv), q.dtype)
    _check((lse, workspace), torch.float32)
    if workspace.numel() * 4 < fa_backward_workspace_bytes(B, H, N, d):
        raise ValueError("workspace smaller than fa_backward_workspace_bytes()")
    fn = getattr(load(), name)
    _call(name, fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                   _ptr(dv), _ptr(workspace), B, H, N, d, float(scale), int(bool(causal)),
                   _stream(stream)))


def fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, stream=None):
    """fa_backward_noalloc on [B, N, H, d] bf16 tensors: fa_backward with the
    library's static scratch in place of a workspace (B*H*N <= 2^21)."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_noalloc", q, {"k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv})
    _lse_shape("fa_backward_noalloc", lse, B, H, N)
    _check((q, k, v, o, do, dq, dk, dv), torch.bfloat16)
    _check((lse,), torch.float32)
    _call("fa_backward_noalloc", load().fa_backward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_backward_single_pass_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_backward_single_pass_workspace_bytes(B, H, N, d))


def fa_backward_single_pass(q, k, v, o, do, lse, dq, dk, dv, workspace, scale: float, causal: bool,
                            stream=None):
    """fa_backward_single_pass on [B, N, H, d] bf16 tensors (workspace: fp32, at least
    fa_backward_single_pass_workspace_bytes())."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_single_pass", q, {"k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv})
    _lse_shape("fa_backward_single_pass", lse, B, H, N)
    _check((q, k, v, o, do, dq, dk, dv), torch.bfloat16)
    _check((lse, workspace), torch.float32)
    if workspace.numel() * 4 < fa_backward_single_pass_workspace_bytes(B, H, N, d):
        raise ValueError("workspace smaller than fa_backward_single_pass_workspace_bytes()")
    _call("fa_backward_single_pass", load().fa_backward_single_pass(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), B, H, N, d, float(scale), int(bool(causal)), _stream(stream)))


def _check_ws(workspace, B, H, N, d):
    if workspace.numel() * 4 < fa_backward_workspace_bytes(B, H, N, d):
        raise ValueError("workspace smaller than fa_backward_workspace_bytes()")


def fa_backward_preprocess(o, do, lse, workspace, stream=None):
    """fa_backward_preprocess: workspace = [-D = -rowsum(dO * O) | -LSE log2(e)] (bf16 tensors)."""
    B, N, H, d = _shape(o)
    _same_shape("fa_backward_preprocess", o, {"do": do})
    _lse_shape("fa_backward_preprocess", lse, B, H, N)
    _check((o, do), torch.bfloat16)
    _check((lse, workspace), torch.float32)
    _check_ws(workspace, B, H, N, d)
    _call("fa_backward_preprocess", load().fa_backward_preprocess(
        _ptr(o), _ptr(do), _ptr(lse), _ptr(workspace), B, H, N, d, _stream(stream)))


def fa_backward_dqdkdv(q, k, v, do, workspace, dq, dk, dv, scale: float, causal: bool, stream=None):
    """fa_backward_dqdkdv: dQ, dK and dV in one launch from the preprocessed workspace."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_dqdkdv", q, {"k": k, "v": v, "do": do, "dq": dq, "dk": dk, "dv": dv})
    _check((q, k, v, do, dq, dk, dv), torch.bfloat16)
    _check((workspace,), torch.float32)
    _check_ws(workspace, B, H, N, d)
    _call("fa_backward_dqdkdv", load().fa_backward_dqdkdv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_backward_dkdv(q, k, v, do, workspace, dk, dv, scale: float, causal: bool, stream=None):
    """fa_backward_dkdv: dK and dV from the preprocessed workspace (bf16 tensors)."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_dkdv", q, {"k": k, "v": v, "do": do, "dk": dk, "dv": dv})
    _check((q, k, v, do, dk, dv), torch.bfloat16)
    _check((workspace,), torch.float32)
    _check_ws(workspace, B, H, N, d)
    _call("fa_backward_dkdv", load().fa_backward_dkdv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace), _ptr(dk), _ptr(dv),
        B, H, N, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_backward_dq(q, k, v, do, workspace, dq, scale: float, causal: bool, stream=None):
    """fa_backward_dq: dQ from the preprocessed workspace (bf16 tensors)."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_dq", q, {"k": k, "v": v, "do": do, "dq": dq})
    _check((q, k, v, do, dq), torch.bfloat16)
    _check((workspace,), torch.float32)
    _check_ws(workspace, B, H, N, d)
    _call("fa_backward_dq", load().fa_backward_dq(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace), _ptr(dq),
        B, H, N, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_decode_splits(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_decode_splits(B, H, Nq, Nk, d))


def fa_decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, splits: int = 0) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits))


def fa_decode(q, k, v, o, lse, workspace, scale: float, causal: bool, splits: int = 0, stream=None):
    """fa_decode: q, o [B, Nq, H, d] and k, v [B, Nk, H, d] bf16; lse [B, H, Nq] fp32."""
    B, Nq, H, d = _shape(q)
    Bk, Nk, Hk, dk = _shape(k)
    if (Bk, Hk, dk) != (B, H, d) or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("fa_decode: q/o and k/v must share B, H and d, k and v the same shape")
    _lse_shape("fa_decode", lse, B, H, Nq)
    _check((q, k, v, o), torch.bfloat16)
    _check((lse, workspace), torch.float32)
    if workspace.numel() * 4 < fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits):
        raise ValueError("workspace smaller than fa_decode_workspace_bytes()")
    _call("fa_decode", load().fa_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), B, H, Nq, Nk, d,
        float(scale), int(bool(causal)), int(splits), _stream(stream)))


def fa_backward_cross(q, k, v, o, do, lse, dq, dk, dv, workspace, scale: float, causal: bool, stream=None):
    """fa_backward_cross: q, o, do, dq [B, Nq, H, d] and k, v, dk, dv [B, Nk, H, d] bf16;
    lse [B, H, Nq] and the workspace fp32."""
    B, Nq, H, d = _shape(q)
    Bk, Nk, Hk, dk_ = _shape(k)
    if (Bk, Hk, dk_) != (B, H, d) or any(tuple(t.shape) != tuple(k.shape) for t in (v, dk, dv)) \
            or any(tuple(t.shape) != tuple(q.shape) for t in (o, do, dq)):
        raise ValueError("fa_backward_cross: q/o/do/dq and k/v/dk/dv must share B, H and d")
    _lse_shape("fa_backward_cross", lse, B, H, Nq)
    _check((q, k, v, o, do, dq, dk, dv), torch.bfloat16)
    _check((lse, workspace), torch.float32)
    if workspace.numel() * 4 < fa_backward_workspace_bytes(B, H, Nq, d):
        raise ValueError("workspace smaller than fa_backward_workspace_bytes(B, H, Nq, d)")
    _call("fa_backward_cross", load().fa_backward_cross(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), B, H, Nq, Nk, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_forward_cross(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    """fa_forward_cross: q, o [B, Nq, H, d] and k, v [B, Nk, H, d] bf16; lse [B, H, Nq] fp32."""
    B, Nq, H, d = _shape(q)
    Bk, Nk, Hk, dk = _shape(k)
    if (Bk, Hk, dk) != (B, H, d) or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("fa_forward_cross: q/o and k/v must share B, H and d, k and v the same shape")
    _lse_shape("fa_forward_cross", lse, B, H, Nq)
    _check((q, k, v, o), torch.bfloat16)
    _check((lse,), torch.float32)
    _call("fa_forward_cross", load().fa_forward_cross(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
        int(bool(causal)), _stream(stream)))


def fa_forward_fp8_workspace_bytes(B: int, H: int, Nk: int, d: int) -> int:
    return int(load().fa_forward_fp8_workspace_bytes(B, H, Nk, d))


_E4M3_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def fa_forward_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, o, lse, workspace,
                   scale: float, causal: bool, stream=None):
    """fa_forward_fp8: q [B, Nq, H, d], k, v [B, Nk, H, d] e4m3 codes (float8_e4m3fn or
    uint8); o [B, Nq, H, d] bf16; lse [B, H, Nq] fp32; workspace a CUDA byte buffer."""
    B, Nq, H, d = _shape(q)
    Bk, Nk, Hk, dk = _shape(k)
    if (Bk, Hk, dk) != (B, H, d) or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("fa_forward_fp8: q/o and k/v must share B, H and d, k and v the same shape")
    _lse_shape("fa_forward_fp8", lse, B, H, Nq)
    for t in (q, k, v):
        if not t.is_cuda or t.dtype not in _E4M3_DTYPES or not t.is_contiguous():
            raise ValueError(f"fa_forward_fp8: expected contiguous e4m3 CUDA tensors, got {t.dtype} on {t.device}")
    _check((o,), torch.bfloat16)
    _check((lse,), torch.float32)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("fa_forward_fp8: workspace must be a contiguous CUDA tensor")
    if workspace.numel() * workspace.element_size() < fa_forward_fp8_workspace_bytes(B, H, Nk, d):
        raise ValueError("workspace smaller than fa_forward_fp8_workspace_bytes()")
    _call("fa_forward_fp8", load().fa_forward_fp8(
        _ptr(q), _ptr(k), _ptr(v), float(q_descale), float(k_descale), float(v_descale), _ptr(o),
        _ptr(lse), _ptr(workspace), B, H, Nq, Nk, d, float(scale), int(bool(causal)), _stream(stream)))


def fa_forward_dropout(q, k, v, o, lse, scale: float, causal: bool, p_drop: float, seed: int, offset: int = 0,
                       stream=None):
    """fa_forward_dropout on [B, N, H, d] bf16 tensors; lse [B, H, N] fp32."""
    B, N, H, d = _shape(q)
    _same_shape("fa_forward_dropout", q, {"k": k, "v": v, "o": o})
    _lse_shape("fa_forward_dropout", lse, B, H, N)
    _check((q, k, v, o), torch.bfloat16)
    _check((lse,), torch.float32)
    _call("fa_forward_dropout", load().fa_forward_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
        float(p_drop), int(seed), int(offset), _stream(stream)))


def fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, workspace, scale: float, causal: bool,
                        p_drop: float, seed: int, offset: int = 0, stream=None):
    """fa_backward_dropout on [B, N, H, d] bf16 tensors (the forward's p_drop, seed, offset)."""
    B, N, H, d = _shape(q)
    _same_shape("fa_backward_dropout", q, {"k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv})
    _lse_shape("fa_backward_dropout", lse, B, H, N)
    _check((q, k, v, o, do, dq, dk, dv), torch.bfloat16)
    _check((lse, workspace), torch.float32)
    if workspace.numel() * 4 < fa_backward_workspace_bytes(B, H, N, d):
        raise ValueError("workspace smaller than fa_backward_workspace_bytes()")
    _call("fa_backward_dropout", load().fa_backward_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), B, H, N, d, float(scale), int(bool(causal)), float(p_drop), int(seed), int(offset),
        _stream(stream)))
