"""Host-side check of the fused backward's task order (no GPU).

The fused dK/dV + dQ launch maps each workgroup id to (pass, head, tile) with
integer arithmetic and a binary search on the task cost.  This re-states that
mapping in Python line for line and checks, for many grid shapes, that it is a
bijection onto every (pass, head, tile) with head < B*H and tile < ntiles, and
that within each XCD group the costs come out in non-increasing order.
"""
import pytest


def cdiv(a, b):
    return a // b      # all operands are non-negative


def fused_task(id_, nt, bhcount, causal):
    if bhcount % 8 == 0:
        group, rank, hpg = id_ & 7, id_ >> 3, bhcount >> 3
    else:
        group, rank, hpg = 0, id_, bhcount
    if not causal:
        is_kv = rank < nt * hpg
        which = rank if is_kv else rank - nt * hpg
        return is_kv, group * hpg + which % hpg, which // hpg

    def count_ge(w):
        kvmax, dqmax = 8 * (2 * nt - 1), 6 * (2 * nt - 1)
        kv = 0 if w > kvmax else min(nt, cdiv(kvmax - w, 16) + 1)
        dq = 0 if w > dqmax else min(nt, cdiv(dqmax - w, 12) + 1)
        return (kv + dq) * hpg

    lo, hi = 1, 8 * (2 * nt - 1)
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if count_ge(mid) > rank:
            lo = mid
        else:
            hi = mid - 1
    w = lo
    pos = rank - count_ge(w + 1)
    is_kv = (w % 16) == 8
    tile = nt - cdiv(cdiv(w, 8) + 1, 2) if is_kv else cdiv(cdiv(w, 6) - 1, 2)
    return is_kv, group * hpg + pos, tile


def cost(is_kv, tile, nt):
    return 8 * (2 * (nt - tile) - 1) if is_kv else 6 * (2 * tile + 1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 7, 32, 64, 65, 256])
@pytest.mark.parametrize("bhcount", [1, 2, 3, 6, 8, 16, 24, 32, 64])
def test_fused_task_is_a_bijection(nt, bhcount, causal):
    grid = 2 * nt * bhcount
    seen = set()
    last = {}
    for i in range(grid):
        is_kv, bh, tile = fused_task(i, nt, bhcount, causal)
        assert 0 <= bh < bhcount and 0 <= tile < nt, (i, is_kv, bh, tile)
        key = (is_kv, bh, tile)
        assert key not in seen, f"task {key} mapped twice"
        seen.add(key)
        if causal:   # heaviest first inside each XCD group
            g = i & 7 if bhcount % 8 == 0 else 0
            c = cost(is_kv, tile, nt)
            assert c <= last.get(g, c), (i, c, last[g])
            last[g] = c
    assert len(seen) == grid


def xcd_remap(id_, count):
    x, slot = id_ & 7, id_ >> 3
    q, r = count >> 3, count & 7
    return x * q + (x if x < r else r) + slot


def tile_of(id_, ntiles, bhcount, causal, heavy_high):
    if bhcount % 8 == 0:
        x, s = id_ & 7, id_ >> 3
        hpx = bhcount >> 3
        if causal:
            bh, rank = x * hpx + s % hpx, s // hpx
        else:
            bh, rank = x * hpx + s // ntiles, s % ntiles
    else:
        L = xcd_remap(id_, ntiles * bhcount)
        bh, rank = L // ntiles, L % ntiles
    return bh, (ntiles - 1 - rank if heavy_high else rank)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heavy_high", [False, True])
@pytest.mark.parametrize("nt", [1, 3, 32, 64, 257])
@pytest.mark.parametrize("bhcount", [1, 3, 6, 8, 16, 32, 40])
def test_tile_of_is_a_bijection(nt, bhcount, causal, heavy_high):
    seen = {tile_of(i, nt, bhcount, causal, heavy_high) for i in range(nt * bhcount)}
    assert len(seen) == nt * bhcount
    assert all(0 <= bh < bhcount and 0 <= t < nt for bh, t in seen)
