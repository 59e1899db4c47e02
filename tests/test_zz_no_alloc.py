"""fa_backward_noalloc (the backward with the library's static scratch in place
of a workspace) against fa_backward, through the C ABI: bitwise equal on two
calls in a row, the second with a smaller input; and the size limit."""
import pytest
import torch

from gpu_helpers import inputs, require_gpu, say

pytestmark = pytest.mark.gpu


def _pair(shape, seed, causal):
    import exact_io_aware_39_amd as fa
    B, N, H, d = shape
    say(f"noalloc backward shape={shape} causal={causal} seed={seed}")
    dev, _ = inputs(shape, "bf16", seed, with_do=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal)
    ref = fa.backward(q, k, v, o, do, lse, scale=scale, causal=causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_backward_noalloc(q, k, v, o, do, lse, *got, scale, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name} of fa_backward_noalloc differs from fa_backward {shape}"


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_backward_twice(causal):
    require_gpu()
    _pair((2, 1000, 4, 64), 31, causal)     # larger first
    _pair((1, 129, 3, 128), 32, causal)     # then smaller: stale scratch must not leak in
    _pair((1, 300, 2, 256), 33, causal)


def test_noalloc_at_the_scratch_limit():
    """B*H*N = 2^21 rows exactly (the array's capacity), against fa_backward."""
    require_gpu()
    _pair((1, 65536, 32, 64), 34, True)


def test_noalloc_rejects_beyond_the_limit():
    require_gpu()
    import exact_io_aware_39_amd as fa
    from exact_io_aware_39_amd._lib import FA_ERR_SCRATCH_LIMIT
    B, N, H, d = 1, 65537, 32, 64
    t = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.fa_backward_noalloc(t, t, t, t, t, lse, t, t, t, 0.125, True)
    assert ei.value.status == FA_ERR_SCRATCH_LIMIT
