"""Host-side model of the split-tail work plan, checked for coverage, merge lists and
wait order over a sweep of grid sizes (no GPU).

The model restates, in Python integer arithmetic, the plan both attention kernels follow when
the last, partial round of query tiles is split over every compute unit (split_tail_plan in
csrc/attn_bf16.hip, split_tail_items, xcd_remap and the empty-range rule of split_merge in
csrc/common.hpp): with U query tiles of nk key tiles on a grid of G workgroups, rounds = U // G
rounds of whole tiles, then T = (U - rounds * G) * nk (query tile, key tile) units cut into
equal ranges [T g / G, T (g + 1) / G), one per workgroup, whose pieces run last tile first.

Invariants (any one failing would give wrong, NaN or hanging output on the GPU):
  * every (query tile, key tile) unit is processed exactly once;
  * a tile processed in pieces has exactly one piece that ends at its last key tile (the
    owner, or the whole tile); every other piece writes a partial;
  * a workgroup writes at most one partial, in its first tail piece, before any wait;
  * the owner merges exactly the workgroups that wrote this tile's partials (workgroups
    with an empty range skipped), all lower-numbered than itself, so waits point down only.
"""
import itertools

import pytest


def plan(U, G, nk, windowed=False):
    """(rounds, tail_units) or None when the split is not taken."""
    if G <= 0 or windowed or U < 3 * G or nk < 2:
        return None
    if U / (-(-U // G) * G) >= 0.95:
        return None
    rounds = U // G
    return rounds, (U - rounds * G) * nk


def xcd_remap(w, n):
    x, slot = w & 7, w >> 3
    q, rem = n >> 3, n & 7
    return x * q + min(x, rem) + slot


def items(g, G, rounds, nk, T):
    """Work items of workgroup g in processing order: (tile, tb, te, mode, p_lo, p_hi)."""
    s0, e0 = T * g // G, T * (g + 1) // G
    base = rounds * G
    u_hi = (e0 - 1) // nk if e0 > s0 else 0
    u_lo = s0 // nk
    n_items = rounds + (u_hi - u_lo + 1 if e0 > s0 else 0)
    out = []
    for it in range(n_items):
        if it < rounds:
            out.append((it * G + xcd_remap(g, G), 0, nk, "full", 0, -1))
            continue
        u = u_hi - (it - rounds)
        ub = u * nk
        tb = max(s0, ub) - ub
        te = min(e0, ub + nk) - ub
        mode, p_lo, p_hi = "full", 0, -1
        if te < nk:
            mode = "partial"
        elif tb > 0:
            mode, p_hi, p_lo = "owner", g - 1, g - 1
            while p_lo > 0 and T * p_lo // G > ub:
                p_lo -= 1
        out.append((base + u, tb, te, mode, p_lo, p_hi))
    return out


def check(U, G, nk):
    p = plan(U, G, nk)
    if p is None:
        return False
    rounds, T = p
    seen = {}
    partial_of = {}  # tile -> set of workgroups that wrote a partial of it
    owners = {}      # tile -> (workgroup, merge list)
    for g in range(G):
        its = items(g, G, rounds, nk, T)
        n_partial = 0
        for k, (L, tb, te, mode, p_lo, p_hi) in enumerate(its):
            assert 0 <= L < U and 0 <= tb < te <= nk, (U, G, nk, g, L, tb, te)
            for t in range(tb, te):
                assert (L, t) not in seen, ("unit twice", U, G, nk, L, t, g, seen[(L, t)])
                seen[(L, t)] = g
            if mode == "partial":
                n_partial += 1
                assert k == rounds, ("partial is not the first tail piece", U, G, nk, g)
                partial_of.setdefault(L, set()).add(g)
            elif mode == "owner":
                assert L not in owners, ("two owners", U, G, nk, L)
                merged = [q for q in range(p_lo, p_hi + 1) if T * q // G != T * (q + 1) // G]
                assert all(q < g for q in merged), ("waits upward", U, G, nk, g, merged)
                owners[L] = (g, merged)
        assert n_partial <= 1, ("two partials in one slot", U, G, nk, g)
    assert len(seen) == U * nk, ("units missed", U, G, nk, U * nk - len(seen))
    for L, writers in partial_of.items():
        assert L in owners, ("partial never merged", U, G, nk, L)
        assert sorted(writers) == owners[L][1], ("merge list", U, G, nk, L, sorted(writers), owners[L][1])
    for L, (g, merged) in owners.items():
        assert merged and set(merged) == partial_of.get(L, set()), ("owner without partials", U, G, nk, L)
    return True


GRIDS = [1, 2, 3, 7, 8, 9, 13, 64, 255, 256, 304]
KEY_TILES = [2, 3, 5, 16, 72]


@pytest.mark.parametrize("G", GRIDS)
def test_plan_invariants(G):
    taken = 0
    for nk in KEY_TILES:
        for U in sorted({3 * G + d for d in (1, 2, G // 3, G // 2, (9 * G) // 10, G - 1)} |
                        {7 * G + G // 4, 19 * G + G // 8}):
            if U > 0:
                taken += check(U, G, nk)
    assert taken > 0 or G < 3


def test_fewer_units_than_workgroups_is_covered():
    # 864 query tiles of 2 key tiles on 256 workgroups: 192 tail units, 64 empty ranges
    rounds, T = plan(864, 256, 2)
    assert (rounds, T) == (3, 192)
    assert sum(T * g // 256 == T * (g + 1) // 256 for g in range(256)) == 64
    assert check(864, 256, 2)


def test_split_not_taken():
    assert plan(432, 256, 72) is None          # FLUX-1024: fewer than three whole rounds
    assert plan(768, 256, 72) is None          # a full last round
    assert plan(1020, 256, 72) is None         # last round 98 % full
    assert plan(864, 256, 1) is None           # one key tile: nothing to split
    assert plan(864, 256, 72, windowed=True) is None
    assert plan(1584, 256, 264) == (6, 48 * 264)  # FLUX-2048
