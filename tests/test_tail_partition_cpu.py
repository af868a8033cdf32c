"""The balanced tail's partition and the persistent launch's work queues (host-side property
checks of their index formulas).

The forward kernels' tail spreads U = n_tail * T units (query tile, key tile) over P runs: run w
takes [floor(U w / P), floor(U (w+1) / P)) and splits it at query-tile boundaries into at most
two segments.  Segment 0 goes to slot w; a segment 1, which starts at the first unit of tail
tile j, to slot P + j - 1.  The fix-up finds the runs of tail tile j starting from
w0 = floor(((jT + 1) P - 1) / U), the last run starting at or before jT, and reads slot
P + j - 1 for the run that started before jT, slot w for the others.  These formulas are
restated here and checked for every case: each unit is computed exactly once, no run has a third
segment, no two segments share a slot, and the fix-up finds exactly the runs that cover each
tile, with the slots the kernel wrote.  P is one run per CU, or up to four when the launch is
persistent.

A persistent launch cuts every tail tile into r equal parts instead (part p of tile j is run
p * n_tail + j, key tiles [T p / r, T (p + 1) / r), slot p * n_tail + j): checked likewise, for
the r the library's rule picks and for forced ones.

A persistent launch of G workgroups gives workgroup g item g first; the other items are dealt
by b % 8 over 8 queues of whole query tiles and 8 of tail runs, and a workgroup takes from its
own XCD's whole-tile queue, the other whole-tile queues, then the tail queues.  Simulated with
workgroups on random XCDs asking in random order: every item is taken exactly once, and no
workgroup takes a whole tile after a tail run.
"""
import itertools
import random

import pytest


def sk_start(U, w, P):
    return U * w // P


def sk_slot(w, seg, j, P):
    return w if seg == 0 else P + j - 1


def kernel_segments(U, T, P, w):
    """(tile, first key tile, key tiles, slot) of run w, as the kernel's segment loop."""
    u0, u1 = sk_start(U, w, P), sk_start(U, w + 1, P)
    out = []
    for seg in itertools.count():
        cut = (u0 // T + 1) * T
        s0 = u0 if seg == 0 else cut
        s1 = (min(u1, cut)) if seg == 0 else u1
        if seg > 1 or s0 >= s1:
            break
        out.append((s0 // T, s0 % T, s1 - s0, sk_slot(w, seg, s0 // T, P)))
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
            slots.append(sk_slot(w, 1 if u0 < t0 else 0, j, P))
        w += 1
    return slots


def plan(n_tail, T, cus=256, runs_per_cu=1):
    U = n_tail * T
    return U, min(cus * runs_per_cu, U)


CASES = [(1, 16), (3, 79), (3, 141), (44, 79), (96, 690), (176, 72), (180, 690), (208, 696), (255, 64), (1, 2000)]
rng = random.Random(7)
CASES += [(rng.randint(1, 255), rng.randint(16, 800)) for _ in range(40)]


@pytest.mark.parametrize("runs_per_cu", [1, 2, 4])
@pytest.mark.parametrize("n_tail,T", CASES)
def test_every_unit_once_and_fixup_finds_the_runs(n_tail, T, runs_per_cu):
    U, P = plan(n_tail, T, runs_per_cu=runs_per_cu)
    assert P > n_tail                      # the launcher's condition: runs of at most T units
    covered = [0] * U
    by_tile = {}
    slots = []
    for w in range(P):
        segs = kernel_segments(U, T, P, w)
        assert len(segs) <= 2
        for tile, g0, n, slot in segs:
            assert 0 <= g0 and g0 + n <= T and n > 0
            for u in range(tile * T + g0, tile * T + g0 + n):
                covered[u] += 1
            by_tile.setdefault(tile, []).append(slot)
            slots.append(slot)
    assert all(c == 1 for c in covered)
    assert len(set(slots)) == len(slots) and 0 <= min(slots) and max(slots) < P + n_tail
    for j in range(n_tail):
        assert sorted(fixup_runs(U, T, P, j)) == sorted(by_tile[j]), j


def test_first_workgroup_formula_is_the_last_start_at_or_before():
    for U, P in itertools.product(range(1, 60), range(1, 40)):
        for x in range(U):
            w = ((x + 1) * P - 1) // U
            assert sk_start(U, w, P) <= x and (w + 1 == P or sk_start(U, w + 1, P) > x)


def part_segments(T, r, n_tail, w):
    """(tile, first key tile, key tiles, slot) of run w of the r-part tail, as the kernel's."""
    p, j = w // n_tail, w % n_tail
    g0, g1 = T * p // r, T * (p + 1) // r
    return [(j, g0, g1 - g0, w)]


def part_fixup_slots(r, n_tail, j):
    return [p * n_tail + j for p in range(r)]


def library_parts(n_tail, T, cus=256, min_run=128, most_per_cu=4):
    """The library's choice of r for a persistent launch (0: runs of equal units): the r <= r_max
    whose parts leave the least of their last round idle (a larger r unless a smaller one is
    better by 0.02), none above 0.3 or with fewer parts than CUs."""
    most = (most_per_cu * cus + n_tail - 1) // n_tail
    r_max = min(T // min_run, most)
    r, best = 0, 0.3
    for c in range(r_max, 1, -1):
        per = c * n_tail / cus
        if per < 1.0:
            break
        idle = -(-(c * n_tail) // cus) / per - 1.0
        if (idle <= best) if r == 0 else (idle < best - 0.02):
            r, best = c, idle
    return r


PART_CASES = [(208, 690, None), (96, 690, None), (180, 690, None), (208, 690, 2), (44, 79, 5), (3, 79, 79),
              (255, 2000, None), (1, 2000, None), (7, 16, 16)]
PART_CASES += [(rng.randint(1, 255), rng.randint(2, 3000), None) for _ in range(20)]


@pytest.mark.parametrize("n_tail,T,forced", PART_CASES)
def test_parts_every_unit_once_and_fixup_finds_them(n_tail, T, forced):
    r = forced or library_parts(n_tail, T)
    if r == 0:
        return
    assert 2 <= r <= T and r * n_tail <= 4 * 256 + n_tail  # fits the workspace's tail room
    covered = [0] * (n_tail * T)
    by_tile = {}
    slots = []
    for w in range(r * n_tail):
        for tile, g0, n, slot in part_segments(T, r, n_tail, w):
            assert n >= 1 and g0 + n <= T
            for u in range(tile * T + g0, tile * T + g0 + n):
                covered[u] += 1
            by_tile.setdefault(tile, []).append(slot)
            slots.append(slot)
    assert all(c == 1 for c in covered)
    assert sorted(slots) == list(range(r * n_tail))
    for j in range(n_tail):
        assert sorted(part_fixup_slots(r, n_tail, j)) == sorted(by_tile[j])


def test_library_parts_at_the_workloads():
    # full sequence, ring share, Ulysses share (bf16): 1040 parts (4.06 per CU), 480 (1.88), 720
    # (2.81; 5 parts would make 3.52); the FP8 kernel's parts are at least 192 key tiles: 624 at
    # the full sequence, none at the Ulysses share (2 or 3 parts per tile leave 42% of the last
    # round idle)
    assert library_parts(208, 690) == 5 and library_parts(96, 690) == 5 and library_parts(180, 690) == 4
    assert library_parts(208, 690, min_run=192) == 3 and library_parts(180, 690, min_run=192) == 0
    assert library_parts(208, 87) == 0  # a ring chunk's launch: runs of equal units
    assert library_parts(96, 690, min_run=170) == 0  # 4 parts: 1.5 per CU, 3 parts: 1.125


def wq_next(counters, xcd, G, n_whole, n_items, empty):
    """The kernel's next item for a workgroup on XCD xcd (counters: the 16 queue counters;
    empty: the set of queues this workgroup found empty)."""
    for k in range(16):
        x = (xcd + k) & 7
        qi = (k & 8) | x
        lo = G if k < 8 else max(G, n_whole)
        hi = n_whole if k < 8 else n_items
        first = lo + ((x - lo) & 7)
        if qi in empty:
            continue
        if first < hi:
            b = first + 8 * counters[qi]
            counters[qi] += 1
            if b < hi:
                return b
        empty.add(qi)
    return -1


QUEUE_CASES = [(256, 2560, 2816), (256, 2768, 2768), (256, 256, 1280), (256, 96, 1120), (256, 352, 352),
               (256, 300, 300), (200, 150, 1000), (256, 257, 257), (256, 0, 1024), (37, 100, 350)]
QUEUE_CASES += [(rng.choice([8, 64, 256, 255]), rng.randint(0, 900), 0) for _ in range(20)]


@pytest.mark.parametrize("G,n_whole,n_items", QUEUE_CASES)
def test_persistent_queues_hand_out_every_item_once(G, n_whole, n_items):
    n_items = max(n_items, n_whole)
    G = min(G, n_items) if n_items else G
    r = random.Random(G * 7919 + n_whole * 31 + n_items)
    counters = [0] * 16
    taken = list(range(min(G, n_items)))           # the first round: workgroup g takes item g
    alive = {g: (r.randrange(8), set(), g >= n_whole) for g in range(min(G, n_items))}
    while alive:
        g = r.choice(list(alive))
        xcd, empty, had_tail = alive[g]
        b = wq_next(counters, xcd, G, n_whole, n_items, empty)
        if b < 0:
            del alive[g]
            continue
        assert not (had_tail and b < n_whole), "a whole tile after a tail run"
        alive[g] = (xcd, empty, had_tail or b >= n_whole)
        taken.append(b)
    assert sorted(taken) == list(range(n_items))
    assert all(c <= n_items + 16 * G for c in counters)  # no runaway counter
