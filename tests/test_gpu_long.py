"""Long sequences beyond the largest workload (N = 2^17 forward, N = 2^16
forward + backward): 64-bit offsets, buffer-descriptor ranges and the causal
task order at sizes where every head spans thousands of tiles.  Checked on
seeded rows (first and last included) against the fp64 oracle, and the
backward's key-side gradients on every key by invariants that hold at any
size."""
import numpy as np
import pytest
import torch

import oracle.attention as ora
from gpu_helpers import check, check_lse, inputs, require_gpu, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import exact_io_aware_39_amd as fa
    fa.load()


def sample_rows(N, seed, count=40):
    rng = np.random.default_rng(seed)
    rows = rng.choice(N, size=count, replace=False)
    return np.unique(np.concatenate([rows, [0, 1, N // 2, N - 2, N - 1]]))


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_forward_n131072(d, causal):
    import exact_io_aware_39_amd as fa
    B, N, H = 1, 1 << 17, 1
    say(f"long forward [{B},{N},{H},{d}] causal={causal}")
    dev, f64 = inputs((B, N, H, d), "bf16", 9100 + d, qk_mult=1.0)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=d ** -0.5, causal=causal)
    torch.cuda.synchronize()
    rows = sample_rows(N, 9200 + d)
    q, k, v = f64["q"][0, :, 0], f64["k"][0, :, 0], f64["v"][0, :, 0]
    o_ref, l_ref = ora.forward_rows(q[rows], rows, k, v, d ** -0.5, causal)
    idx = torch.as_tensor(rows, device="cuda")
    e = check(to64(o[0, idx, 0]), o_ref, "bf16", f"O long d={d}")
    check_lse(to64(lse[0, 0, idx]), l_ref, f"LSE long d={d}")
    say(f"  ok: O max/mean abs err {e}")


def test_backward_n65536():
    import exact_io_aware_39_amd as fa
    B, N, H, d = 1, 1 << 16, 2, 64
    scale = 0.125
    say(f"long backward [{B},{N},{H},{d}] causal=True")
    dev, f64 = inputs((B, N, H, d), "bf16", 9300, with_do=True)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=scale, causal=True)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(N, 9301)
    idx = torch.as_tensor(rows, device="cuda")
    for h in range(H):
        q, k, v, do = (f64[n][0, :, h] for n in ("q", "k", "v", "do"))
        # dQ of a row needs only that row's P and dP: the oracle on the sampled rows
        dq_ref, _, _, _ = ora.backward(q[rows], k, v, do[rows], scale, True, rows=rows)
        check(to64(dq[0, idx, h]), dq_ref, "bf16", f"dQ long h={h}")
        # every key: sum_j dV_j = sum_i dO_i (rows of P sum to one) and
        # sum_j dK_j = 0 (softmax is shift invariant), within the rounding of
        # N bf16 rows
        sv = dv[0, :, h].double().sum(dim=0).cpu().numpy()
        so = dev["do"][0, :, h].double().sum(dim=0).cpu().numpy()
        sk = dk[0, :, h].double().sum(dim=0).cpu().numpy()
        bound_v = 5 * 2 * 2.0 ** -8 / np.sqrt(3) * float(np.sqrt((to64(dv[0, :, h]) ** 2).sum(axis=0)).max()) + 1e-6
        bound_k = 5 * 2 * 2.0 ** -8 / np.sqrt(3) * float(np.sqrt((to64(dk[0, :, h]) ** 2).sum(axis=0)).max()) + 1e-6
        assert np.abs(sv - so).max() <= bound_v, f"sum dV h={h}: {np.abs(sv - so).max()} > {bound_v}"
        assert np.abs(sk).max() <= bound_k, f"sum dK h={h}: {np.abs(sk).max()} > {bound_k}"
    say("  ok")
