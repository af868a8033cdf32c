"""The balanced tail's partition (host-side property check of its index formulas).

The bf16 kernel's tail spreads U = n_tail * T units (query tile, key tile) over P workgroups:
workgroup w takes [floor(U w / P), floor(U (w+1) / P)) and splits it at query-tile boundaries
into at most two segments, segment i going to slot 2w + i.  The fix-up finds the runs of tail
tile j starting from w0 = floor(((jT + 1) P - 1) / U), the last workgroup starting at or before
jT, and reads slot 2w + (1 if the run started before jT else 0).  These formulas are restated
here and checked for every case: each unit is computed exactly once, no run has a third
segment, and the fix-up finds exactly the runs that cover each tile, with the slots the kernel
wrote.
"""
import itertools
import random

import pytest


def sk_start(U, w, P):
    return U * w // P


def kernel_segments(U, T, P, w):
    """(tile, first key tile, key tiles, slot) of workgroup w, as the kernel's segment loop."""
    u0, u1 = sk_start(U, w, P), sk_start(U, w + 1, P)
    out = []
    for seg in itertools.count():
        cut = (u0 // T + 1) * T
        s0 = u0 if seg == 0 else cut
        s1 = (min(u1, cut)) if seg == 0 else u1
        if seg > 1 or s0 >= s1:
            break
        out.append((s0 // T, s0 % T, s1 - s0, 2 * w + seg))
    return out


def fixup_runs(U, T, P, j):
    """Slots the fix-up merges for tail tile j, as its loop."""
    t0, t1 = j * T, (j + 1) * T
    w = ((t0 + 1) * P - 1) // U
    slots = []
    while w < P:
        u0, u1 = sk_start(U, w, P), sk_start(U, w + 1, P)
        if u0 >= t1:
            break
        if u1 != u0:
            slots.append(2 * w + (1 if u0 < t0 else 0))
        w += 1
    return slots


def plan(n_tail, T, cus=256):
    U = n_tail * T
    return U, min(cus, U)


CASES = [(1, 16), (3, 79), (3, 141), (44, 79), (96, 690), (176, 72), (180, 690), (208, 696), (255, 64), (1, 2000)]
rng = random.Random(7)
CASES += [(rng.randint(1, 255), rng.randint(16, 800)) for _ in range(40)]


@pytest.mark.parametrize("n_tail,T", CASES)
def test_every_unit_once_and_fixup_finds_the_runs(n_tail, T):
    U, P = plan(n_tail, T)
    assert P > n_tail                      # the launcher's condition: runs of at most T units
    covered = [0] * U
    by_tile = {}
    for w in range(P):
        segs = kernel_segments(U, T, P, w)
        assert len(segs) <= 2
        for tile, g0, n, slot in segs:
            assert 0 <= g0 and g0 + n <= T and n > 0
            for u in range(tile * T + g0, tile * T + g0 + n):
                covered[u] += 1
            by_tile.setdefault(tile, []).append(slot)
    assert all(c == 1 for c in covered)
    for j in range(n_tail):
        assert sorted(fixup_runs(U, T, P, j)) == sorted(by_tile[j]), j


def test_first_workgroup_formula_is_the_last_start_at_or_before():
    for U, P in itertools.product(range(1, 60), range(1, 40)):
        for x in range(U):
            w = ((x + 1) * P - 1) // U
            assert sk_start(U, w, P) <= x and (w + 1 == P or sk_start(U, w + 1, P) > x)
