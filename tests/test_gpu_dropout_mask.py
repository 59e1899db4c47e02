"""Bit-exact check of the dropout keep mask that each pass draws on the GPU.

The mask is integer work (16-bit fields of Philox4x32-10 outputs compared with
round(p 2^16)), so it is compared bit for bit with oracle.dropout.keep_mask,
not through a float tolerance.  Inputs are chosen so that every kept or dropped element shows up
in its own output element (N <= d, Q = 0 so that every visible key of row i
has the probability 1 / n_i, n_i = number of keys row i sees):

* forward, V = identity (row j of V is e_j): O_ij = z_ij / n_i, which is
  exactly zero when key j of row i is dropped and at least 1 / N otherwise;
* dK/dV pass, dO = identity: dV_ji = P_ij z_ij, again exactly zero when
  dropped (this is the pass whose lanes trade keep bits across the 8 lanes
  of one generator call at d <= 128);
* dQ pass, V = all ones, dO = identity, K = identity: dP_ij = 1, so
  dS_ij = P_ij (z_ij - D_i) and dQ_ij = dS_ij; a kept element gives
  P_i (s - D_i), a dropped one -P_i D_i (s = keep_scale(p), D_i read from the
  GPU's own O), two values s P_i apart, and the element is classified by the
  midpoint between them.

Where row i cannot see key j (causal) every one of these outputs must be 0.
A single flipped keep bit changes one recovered element, so any mismatch
with the oracle's mask fails the test.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_39_amd as fa
import oracle.dropout as drop
from gpu_helpers import require_gpu, say, to64

pytestmark = pytest.mark.gpu


def _identity_rows(B, N, H, d):
    """[B, N, H, d] bf16 tensor whose row j of every head is e_j (N <= d)."""
    x = torch.zeros((B, N, H, d), dtype=torch.float32)
    idx = torch.arange(N)
    x[:, idx, :, idx] = 1.0
    return x.to(torch.bfloat16).cuda()


def _visible(N, causal):
    if not causal:
        return np.ones((N, N), dtype=bool)
    return np.arange(N)[None, :] <= np.arange(N)[:, None]


def _read_masks(B, H, N, d, causal, p, seed, offset):
    """The keep masks recovered from the forward, the dK/dV pass and the dQ
    pass, as boolean [B*H, N, N] arrays (row, key), and the visibility."""
    assert N <= d
    scale = 0.5                      # any: Q = 0 makes every score 0
    zero = torch.zeros((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    eye = _identity_rows(B, N, H, d)
    ones = torch.ones((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    vis = _visible(N, causal)
    n = vis.sum(axis=1).astype(np.float64)              # keys seen by each row
    s = float(np.float32(drop.keep_scale(p)))

    # forward and dK/dV pass: V = identity, dO = identity
    o, lse = fa.forward_dropout(zero, eye, eye, p, seed, offset, scale=scale, causal=causal)
    _, _, dv = fa.backward_dropout(zero, eye, eye, o, eye, lse, p, seed, offset, scale=scale, causal=causal)
    # dQ pass: V = ones, dO = identity, K = identity
    o1, lse1 = fa.forward_dropout(zero, eye, ones, p, seed, offset, scale=scale, causal=causal)
    dq, _, _ = fa.backward_dropout(zero, eye, ones, o1, eye, lse1, p, seed, offset, scale=1.0, causal=causal)
    torch.cuda.synchronize()
    o64, dv64, dq64, o164 = to64(o), to64(dv), to64(dq), to64(o1)

    fwd, dkdv, dqm = (np.zeros((B * H, N, N), dtype=bool) for _ in range(3))
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            O = o64[b, :, h, :N]                         # [row, key]
            dVt = dv64[b, :, h, :N].T                    # dV[key, row] -> [row, key]
            dQ = dq64[b, :, h, :N]                       # [row, key]
            D = np.diag(o164[b, :, h, :N])               # D_i = O_ii (dO = identity)
            for name, x in (("O", O), ("dV", dVt), ("dQ", dQ)):
                assert np.isfinite(x).all(), f"{name}: non-finite (bh={bh})"
                assert (x[~vis] == 0).all(), f"{name}: nonzero where the row cannot see the key (bh={bh})"
            fwd[bh] = vis & (O != 0)
            dkdv[bh] = vis & (dVt != 0)
            mid = (s / 2.0 - D)[:, None] / n[:, None]    # midpoint of P_i (s - D_i) and -P_i D_i
            dqm[bh] = vis & (dQ > mid)
    return fwd, dkdv, dqm, vis


CASES = [
    # d, N, causal, p, seed, offset
    (64, 64, True, 0.1, 0x5EED_0000_1234_ABCD, 0),
    (64, 64, False, 0.5, 1, 3),
    (64, 45, True, 0.9, 0xFFFF_FFFF_FFFF_FFFF, 7),
    (128, 128, False, 0.1, 42, 0),
    (128, 128, True, 0.5, 0x1234_5678_9ABC_DEF0, 11),
    (128, 100, False, 0.25, 99, 1),
    (256, 256, True, 0.1, 2024, 0),
    (256, 256, False, 0.5, 7, 5),
    (256, 200, True, 0.75, 0xDEAD_BEEF, 2),
]


@pytest.mark.parametrize("d,N,causal,p,seed,offset", CASES)
def test_keep_mask_bit_exact(d, N, causal, p, seed, offset):
    require_gpu()
    B, H = 2, 3
    say(f"dropout mask d={d} N={N} causal={causal} p={p} seed={seed:#x} offset={offset}")
    fwd, dkdv, dqm, vis = _read_masks(B, H, N, d, causal, p, seed, offset)
    for bh in range(B * H):
        ref = drop.keep_mask(bh, np.arange(N), N, p, seed, offset) & vis
        for name, got in (("forward", fwd[bh]), ("dK/dV pass", dkdv[bh]), ("dQ pass", dqm[bh])):
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (f"{name}: {len(bad)} keep bits differ from the oracle (bh={bh}), "
                                   f"first at (row, key) = {tuple(bad[0])}")
    kept = np.mean([drop.keep_mask(bh, np.arange(N), N, p, seed, offset)[vis].mean() for bh in range(B * H)])
    say(f"  ok: masks equal bit for bit; kept fraction {kept:.3f} (1 - p = {1 - p:.3f})")
