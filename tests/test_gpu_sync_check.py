"""Race check: every entry point of libfa.so against its sync-check build.

libfa_synccheck.so is built from the same sources with -DFA_SYNC_CHECK: every
asm-issued LDS read and every global/buffer -> LDS copy completes before the
next instruction, and every workgroup barrier first drains all of the wave's
memory operations.  The arithmetic is the same, so where the normal build's
ordering is right (each tile read after its copy landed and after the
barrier that publishes it, no copy into a buffer another wave still reads, no
asm read used before its wait) the two builds give the same bits.  A race in
the normal build shows as a difference here.  dQ of the single-pass backward
is summed in fp32 with atomics in an order that varies from run to run and
then rounded to bf16, so it may differ by one bf16 unit in the last place
(2^-7 relative, plus 1e-5 absolute for the fp32 sum near zero); every other
output is compared bit for bit.

Shapes are ragged (partial last tiles) and span several tiles, causal and
not, for every head size each entry point supports.
"""
import pytest
import torch

import exact_io_aware_39_amd as fa
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _libs():
    require_gpu()
    fa.load()
    fa.load(fa.SYNC_CHECK_LIB_PATH)


def _rand(shape, seed, dtype=torch.bfloat16, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(dtype).cuda()


def _both(run):
    """run() under libfa.so and under the sync-check build; returns both
    tuples of output tensors."""
    a = run()
    torch.cuda.synchronize()
    with fa.use_library(fa.SYNC_CHECK_LIB_PATH):
        b = run()
        torch.cuda.synchronize()
    return a, b


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _same(a, b, names, loose=()):
    for name, x, y in zip(names, a, b):
        if name in loose:
            tol = 2.0 ** -7 * torch.maximum(x.float().abs(), y.float().abs()) + 1e-5
            bad = ((x.float() - y.float()).abs() > tol).sum().item()
            assert bad == 0, f"{name}: {bad} elements differ by more than one bf16 unit between the builds"
            continue
        diff = (_bits(x) != _bits(y)).sum().item()
        assert diff == 0, f"{name}: {diff} bytes differ between the normal and the sync-check build"


SHAPES = [
    (2, 300, 3, 64),
    (2, 300, 3, 128),
    (1, 1100, 8, 64),
    (1, 1100, 8, 128),
    (1, 200, 2, 256),
    (1, 600, 2, 256),
    (2, 4096, 16, 256),   # the 8-wave form of the d = 256 forward (512 workgroups)
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_forward_backward(shape, causal):
    B, N, H, d = shape
    say(f"sync check forward/backward shape={shape} causal={causal}")
    q, k, v, do = (_rand(shape, 100 + i) for i in range(4))
    a, b = _both(lambda: fa.forward(q, k, v, causal=causal))
    _same(a, b, ("O", "LSE"))
    o, lse = a
    a, b = _both(lambda: fa.backward(q, k, v, o, do, lse, causal=causal))
    _same(a, b, ("dQ", "dK", "dV"))
    if d <= 128:
        a, b = _both(lambda: fa.backward_single_pass(q, k, v, o, do, lse, causal=causal))
        _same(a, b, ("dQ single-pass", "dK single-pass", "dV single-pass"), loose=("dQ single-pass",))
    if B * H * N <= 1 << 21:
        def noalloc():
            dq, dk, dv = (torch.empty_like(q) for _ in range(3))
            fa.fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, d ** -0.5, causal)
            return dq, dk, dv
        a, b = _both(noalloc)
        _same(a, b, ("dQ noalloc", "dK noalloc", "dV noalloc"))
    if d == 256:
        # the separate passes (eight-wave pair tiles at this head size)
        def separate():
            ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device="cuda")
            dq, dk, dv = (torch.empty_like(q) for _ in range(3))
            fa.fa_backward_preprocess(o, do, lse, ws)
            fa.fa_backward_dkdv(q, k, v, do, ws, dk, dv, d ** -0.5, causal)
            fa.fa_backward_dq(q, k, v, do, ws, dq, d ** -0.5, causal)
            return dq, dk, dv
        a, b = _both(separate)
        _same(a, b, ("dQ separate", "dK separate", "dV separate"))
    say("  ok: bit-identical")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_decode(d, causal):
    say(f"sync check cross/decode d={d} causal={causal}")
    B, H, Nq, Nk = 2, 3, 130, 333
    q, do = _rand((B, Nq, H, d), 7), _rand((B, Nq, H, d), 8)
    k, v = _rand((B, Nk, H, d), 9), _rand((B, Nk, H, d), 10)
    a, b = _both(lambda: fa.forward_cross(q, k, v, causal=causal))
    _same(a, b, ("O cross", "LSE cross"))
    o, lse = a
    a, b = _both(lambda: fa.backward_cross(q, k, v, o, do, lse, causal=causal))
    _same(a, b, ("dQ cross", "dK cross", "dV cross"))
    for nq in (1, 5, 32):
        qd = _rand((B, nq, H, d), 11 + nq)
        kd, vd = _rand((B, 1500, H, d), 12), _rand((B, 1500, H, d), 13)
        a, b = _both(lambda: fa.decode(qd, kd, vd, causal=causal))
        _same(a, b, (f"O decode Nq={nq}", f"LSE decode Nq={nq}"))
    say("  ok: bit-identical")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_dropout_f32(d, causal):
    say(f"sync check fp8/dropout/f32 d={d} causal={causal}")
    shape = (2, 300, 3, d)
    q8, k8, v8 = (_rand(shape, 20 + i, torch.float32).to(torch.float8_e4m3fn) for i in range(3))
    a, b = _both(lambda: fa.forward_fp8(q8, k8, v8, descales=(0.5, 0.75, 1.25), causal=causal))
    _same(a, b, ("O fp8", "LSE fp8"))
    q, k, v, do = (_rand(shape, 30 + i) for i in range(4))
    a, b = _both(lambda: fa.forward_dropout(q, k, v, 0.2, 1234, 5, causal=causal))
    _same(a, b, ("O dropout", "LSE dropout"))
    o, lse = a
    a, b = _both(lambda: fa.backward_dropout(q, k, v, o, do, lse, 0.2, 1234, 5, causal=causal))
    _same(a, b, ("dQ dropout", "dK dropout", "dV dropout"))
    q, k, v, do = (_rand(shape, 40 + i, torch.float32) for i in range(4))
    a, b = _both(lambda: fa.forward(q, k, v, causal=causal))
    _same(a, b, ("O f32", "LSE f32"))
    o, lse = a
    a, b = _both(lambda: fa.backward(q, k, v, o, do, lse, causal=causal))
    _same(a, b, ("dQ f32", "dK f32", "dV f32"))
    say("  ok: bit-identical")
