"""Fused, IO-aware exact attention for MI355X (gfx950), behind the C ABI of libfa.so.

    o, lse = forward(q, k, v, scale=None, causal=False)
    dq, dk, dv = backward(q, k, v, o, do, lse, scale=None, causal=False)
    o, lse = forward_cross(q, k, v, scale=None, causal=False)      # q: [B, Nq, H, d], k: [B, Nk, H, d]
    dq, dk, dv = backward_cross(q, k, v, o, do, lse, scale=None, causal=False)
    o, lse = decode(q, k, v, scale=None, causal=False, splits=0)   # q: [B, Nq, H, d], Nq <= 32
    o, lse = forward_fp8(q8, k8, v8, descales=(1, 1, 1), scale=None, causal=False)   # e4m3 inputs
    o, lse = forward_dropout(q, k, v, p_drop, seed, offset=0, scale=None, causal=False)
    dq, dk, dv = backward_dropout(q, k, v, o, do, lse, p_drop, seed, offset=0, scale=None, causal=False)

Tensors are contiguous [B, N, H, d] bf16 (or fp32) CUDA tensors with d in
{64, 128} (bf16 forward and backward also 256); lse is fp32 [B, H, N].  scale defaults to d**-0.5, as in the PyTorch
module on the page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org).
PyTorch only supplies device memory and the current stream: every step runs in
the HIP kernels of libfa.so.
"""
from __future__ import annotations

import torch

from ._lib import (FaError, LIB_PATH, SYNC_CHECK_LIB_PATH, use_library, fa_backward, fa_backward_cross, fa_backward_dkdv,  # noqa: F401
                   fa_backward_dq, fa_backward_dqdkdv,
                   fa_backward_preprocess, fa_backward_workspace_bytes, fa_decode,
                   fa_decode_splits, fa_decode_workspace_bytes, fa_forward, fa_forward_cross,
                   fa_forward_fp8, fa_forward_fp8_workspace_bytes, fa_status_string, load,
                   fa_forward_dropout, fa_backward_dropout, fa_backward_single_pass,
                   fa_backward_single_pass_workspace_bytes, fa_backward_noalloc)


def _scale(q, scale):
    return float(q.shape[-1]) ** -0.5 if scale is None else float(scale)


def forward(q, k, v, scale=None, causal=False, stream=None):
    """O and LSE of exact attention; allocates the outputs on q's device."""
    B, N, H, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_forward(q, k, v, o, lse, _scale(q, scale), causal, stream)
    return o, lse


def forward_cross(q, k, v, scale=None, causal=False, stream=None):
    """O and LSE of Nq query rows against Nk keys; with causal=True the rows are
    the last Nq positions of the sequence.  Allocates the outputs."""
    B, Nq, H, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_forward_cross(q, k, v, o, lse, _scale(q, scale), causal, stream)
    return o, lse


def backward(q, k, v, o, do, lse, scale=None, causal=False, stream=None):
    """dQ, dK, dV of sum(O * dO); allocates the outputs and the workspace."""
    B, N, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=q.device)
    fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws, _scale(q, scale), causal, stream)
    return dq, dk, dv


def backward_single_pass(q, k, v, o, do, lse, scale=None, causal=False, stream=None):
    """dQ, dK, dV of sum(O * dO) by the single-pass backward (dQ accumulated
    with fp32 atomics); allocates the outputs and the workspace."""
    B, N, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_backward_single_pass_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32,
                     device=q.device)
    fa_backward_single_pass(q, k, v, o, do, lse, dq, dk, dv, ws, _scale(q, scale), causal, stream)
    return dq, dk, dv


def backward_cross(q, k, v, o, do, lse, scale=None, causal=False, stream=None):
    """dQ, dK, dV of sum(O * dO) for forward_cross (Nq query rows against Nk
    keys); allocates the outputs and the workspace."""
    B, Nq, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_backward_workspace_bytes(B, H, Nq, d) // 4, dtype=torch.float32, device=q.device)
    fa_backward_cross(q, k, v, o, do, lse, dq, dk, dv, ws, _scale(q, scale), causal, stream)
    return dq, dk, dv


def decode(q, k, v, scale=None, causal=False, splits=0, stream=None):
    """O and LSE of a few query rows ([B, Nq, H, d]) against K/V ([B, Nk, H, d]);
    with causal=True the rows are the last Nq positions of the sequence.
    Allocates the outputs and the split workspace."""
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits) // 4),
                     dtype=torch.float32, device=q.device)
    fa_decode(q, k, v, o, lse, ws, _scale(q, scale), causal, splits, stream)
    return o, lse


def forward_fp8(q, k, v, descales=(1.0, 1.0, 1.0), scale=None, causal=False, stream=None):
    """O (bf16) and LSE of e4m3 inputs (float8_e4m3fn or uint8 codes, [B, N, H, d]);
    `descales` = (q, k, v) multipliers of the code values.  q may have fewer rows
    than k and v (causal: the last rows of the sequence).  Allocates the outputs
    and the V^T workspace."""
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    o = torch.empty((B, Nq, H, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa_forward_fp8_workspace_bytes(B, H, Nk, d)), dtype=torch.uint8, device=q.device)
    fa_forward_fp8(q, k, v, *descales, o, lse, ws, _scale(q, scale), causal, stream)
    return o, lse


def forward_dropout(q, k, v, p_drop, seed, offset=0, scale=None, causal=False, stream=None):
    """O and LSE with dropout p_drop on the probabilities (mask from (seed, offset));
    allocates the outputs."""
    B, N, H, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_forward_dropout(q, k, v, o, lse, _scale(q, scale), causal, p_drop, seed, offset, stream)
    return o, lse


def backward_dropout(q, k, v, o, do, lse, p_drop, seed, offset=0, scale=None, causal=False, stream=None):
    """dQ, dK, dV for forward_dropout with the same (p_drop, seed, offset)."""
    B, N, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=q.device)
    fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, _scale(q, scale), causal, p_drop, seed, offset,
                        stream)
    return dq, dk, dv
