"""The merge rule of the balance kernel, checked on the CPU.

The balanced layout's plan ends by merging shed pieces (planning order) into
destination ranks (ascending, each with some room and at most B slots).  The
rule as stated (MoonEP article, section 1: redundant experts planned online;
the greedy itself is the reading taken for it) is sequential: each piece goes
to the current destination as far as its room allows, one slot per (piece,
destination) part, and a destination closes when its room or its slots run
out.  The kernel computes the same thing in parallel: laid end to end, pieces
and rooms both cover [0, T), and a replica is a non-empty overlap of one
piece's span with one destination's span, in stream order; when some
destination would need more than B slots the kernel runs the sequential loop
instead.  This test states both forms plainly and checks, on random plans,
that the parallel form equals the sequential one whenever it applies and that
it declines only when a destination really exceeds B slots.
"""
from __future__ import annotations

import bisect
import random


def sequential(amounts, experts, dests, rooms, B):
    """Replicas (expert, amount, dest, slot) and, per expert, (first, count, moved)."""
    reps, per_expert = [], {}
    if not amounts:
        return reps, per_expert
    pc, di, first, moved, slots = 0, 0, 0, 0, 0
    left, room = amounts[0], rooms[0] if dests else 0
    while pc < len(amounts):
        if di >= len(dests):
            break
        take = min(left, room)
        reps.append((experts[pc], take, dests[di], slots))
        slots += 1
        room -= take
        left -= take
        moved += take
        if room == 0 or slots == B:
            di += 1
            slots = 0
            room = rooms[di] if di < len(dests) else 0
        if left == 0:
            per_expert[experts[pc]] = (first, len(reps) - first, moved)
            pc += 1
            first, moved = len(reps), 0
            left = amounts[pc] if pc < len(amounts) else 0
    if pc < len(amounts) and moved > 0:
        per_expert[experts[pc]] = (first, len(reps) - first, moved)
    return reps, per_expert


def parallel(amounts, experts, dests, rooms, B):
    """The overlap form; None where it declines (totals differ or > B slots)."""
    A = [sum(amounts[:i]) for i in range(len(amounts))]
    C = [sum(rooms[:i]) for i in range(len(rooms))]
    T = sum(amounts)
    if T != sum(rooms):
        return None
    M = len(A) + len(C)
    mval = [None] * M
    for p, a in enumerate(A):       # ties: piece start first
        mval[p + bisect.bisect_left(C, a)] = a
    for d, c in enumerate(C):
        mval[d + bisect.bisect_right(A, c)] = c
    lens = [(mval[j + 1] if j + 1 < M else T) - mval[j] for j in range(M)]
    mrep, n = [], 0
    for ln in lens:
        mrep.append(n)
        n += ln > 0
    reps = [None] * n
    for j in range(M):
        if lens[j] > 0:
            d = bisect.bisect_right(C, mval[j]) - 1
            slot = mrep[j] - mrep[d + bisect.bisect_right(A, C[d])]
            if slot >= B:
                return None
            p = bisect.bisect_right(A, mval[j]) - 1
            reps[mrep[j]] = (experts[p], lens[j], dests[d], slot)
    per_expert = {}
    for p in range(len(A)):
        first = mrep[p + bisect.bisect_left(C, A[p])]
        nxt = mrep[p + 1 + bisect.bisect_left(C, A[p + 1])] if p + 1 < len(A) else n
        per_expert[experts[p]] = (first, nxt - first, amounts[p])
    return reps, per_expert


def _split(rng, total, k):
    cuts = sorted(rng.sample(range(1, total), k - 1)) if k > 1 else []
    b = [0] + cuts + [total]
    return [b[i + 1] - b[i] for i in range(k)]


def test_parallel_merge_equals_sequential():
    rng = random.Random(20261203)
    applied = declined = 0
    for _ in range(20000):
        npiece, ndest = rng.randint(1, 12), rng.randint(1, 8)
        T = rng.randint(max(npiece, ndest), 60)
        amounts, rooms = _split(rng, T, npiece), _split(rng, T, ndest)
        experts = rng.sample(range(100), npiece)
        dests = sorted(rng.sample(range(64), ndest))
        B = rng.randint(1, 6)
        par = parallel(amounts, experts, dests, rooms, B)
        if par is None:
            declined += 1
            unlimited = sequential(amounts, experts, dests, rooms, 10 ** 9)[0]
            per_dest = {}
            for r in unlimited:
                per_dest[r[2]] = per_dest.get(r[2], 0) + 1
            assert max(per_dest.values()) > B
        else:
            applied += 1
            assert par == sequential(amounts, experts, dests, rooms, B)
    assert applied > 5000 and declined > 5000


def test_parallel_merge_hand_example():
    # pieces 5, 3 (experts 7, 9); rooms 4, 4 (ranks 2, 5): breakpoints 0, 4, 5
    reps, per_expert = parallel([5, 3], [7, 9], [2, 5], [4, 4], 4)
    assert reps == [(7, 4, 2, 0), (7, 1, 5, 0), (9, 3, 5, 1)]
    assert per_expert == {7: (0, 2, 5), 9: (2, 1, 3)}
    assert (reps, per_expert) == sequential([5, 3], [7, 9], [2, 5], [4, 4], 4)
    # one slot per destination: rank 5 would need two -> the parallel form declines
    assert parallel([5, 3], [7, 9], [2, 5], [4, 4], 1) is None
