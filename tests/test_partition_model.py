"""The split path's work partition, as a CPU model of what every workgroup of the split kernel
computes (host logic; no GPU).

All rows of all units (sequence b, KV head, head tile), concatenated, are cut into N equal
shares; workgroup w walks rows [w T / N, (w + 1) T / N) and leaves one partial per unit it
crosses, in slot w + u. The combine reads, for unit u, the slots of every workgroup from the
one holding the unit's first row to the one holding its last. These tests check, over random
batches with empty and out-of-range sequences, short and long ones, more workgroups than rows
and both sequence searches the kernel uses (a binary search over the prefix for large batches,
the last lane whose prefix is at most the first row for batches of at most one wave):
  * every row of every valid unit is attended exactly once, and invalid sequences not at all;
  * the partial slots are distinct and fit the workspace's N + units slots;
  * every workgroup between a unit's first and last leaves a partial for it (a segment, or the
    empty partial of a share that holds no rows), which is what the combine assumes.
"""
import random

import pytest


def attended_len(L, append_cap):
    return L + 1 if append_cap > 0 and 0 <= L < append_cap else L


def unit_rows(L, max_len, nq):
    return L if (L >= 1 and L >= nq and L <= max_len) else 0


def prefix(stored, max_len, nq, append_cap, upb):
    pre = [0]
    for L in stored:
        pre.append(pre[-1] + unit_rows(attended_len(L, append_cap), max_len, nq) * upb)
    return pre


def search_binary(pre, pos):
    """The LDS form: the last b with pre[b] <= pos, by bisection over pre[0..batch]."""
    lo, hi = 0, len(pre) - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if pre[mid] <= pos:
            lo = mid
        else:
            hi = mid
    return lo


def search_lanes(pre, pos):
    """The lanes form: lane b holds pre[b]; the ballot of pre[b] <= pos is a prefix of the
    lanes, and its highest set lane is the sequence."""
    mask = 0
    for b in range(len(pre) - 1):
        if pre[b] <= pos:
            mask |= 1 << b
    return mask.bit_length() - 1


def walk(w, N, stored, max_len, nq, append_cap, upb, search, pre=None):
    """Segments (b, ul, r0, r1, slot) of workgroup w, and the unit of its empty share (or None)."""
    pre = pre or prefix(stored, max_len, nq, append_cap, upb)
    T = pre[-1]
    pos, end = w * T // N, (w + 1) * T // N
    segs, empty_unit = [], None
    b, L, ul, row = 0, 1, 0, 0
    if pos < T:
        b = search(pre, pos)
        L = attended_len(stored[b], append_cap)
        off = pos - pre[b]
        ul, row = off // L, off % L
        if pos == end and row > 0:
            empty_unit = b * upb + ul
    while pos < end:
        r0, r1 = row, min(L, row + (end - pos))
        segs.append((b, ul, r0, r1, w + b * upb + ul))
        pos += r1 - r0
        row = 0
        ul += 1
        if ul == upb and pos < end:
            ul = 0
            while True:  # sequences without rows are skipped
                b += 1
                L = attended_len(stored[b], append_cap)
                if unit_rows(L, max_len, nq):
                    break
    return segs, empty_unit


def draw_case(rng):
    B = rng.choice([1, 2, 3, 5, 16, 63, 64, 65, 70])
    max_len = rng.choice([1, 7, 64, 300])
    nq = rng.choice([1, 1, 2, 4])
    append_cap = rng.choice([0, 0, max_len])
    stored = []
    for _ in range(B):
        kind = rng.random()
        if kind < 0.15:
            stored.append(0)
        elif kind < 0.2:
            # no append: out of range; an append into a full cache: flagged, attended as stored
            stored.append(-1 if append_cap == 0 else max_len)
        elif kind < 0.3:
            stored.append(max_len + 5)
        else:
            stored.append(rng.randint(1, max_len))
    upb = rng.choice([1, 2, 3, 8])
    T = prefix(stored, max_len, nq, append_cap, upb)[-1]
    # more workgroups than rows (empty shares) where the batch is small
    N = rng.choice([1, 2, 7, 64, 256, 512] + ([max(1, T), max(1, T // 3), T + 5] if T <= 2000 else []))
    return stored, max_len, nq, append_cap, upb, N


def check_case(stored, max_len, nq, append_cap, upb, N):
    B = len(stored)
    units = B * upb
    pre = prefix(stored, max_len, nq, append_cap, upb)
    per_w = [walk(w, N, stored, max_len, nq, append_cap, upb, search_binary, pre) for w in range(N)]
    # the lanes search finds the same sequence wherever a share starts inside the rows
    for w in range(N):
        pos = w * pre[-1] // N
        if pos < pre[-1]:
            assert search_lanes(pre, pos) == search_binary(pre, pos), (w, pos)
    covered = {}
    slots = set()
    first, last, present = {}, {}, {}
    for w, (segs, empty_unit) in enumerate(per_w):
        for b, ul, r0, r1, slot in segs:
            u = b * upb + ul
            assert slot not in slots and slot < N + units
            slots.add(slot)
            covered.setdefault(u, []).append((r0, r1))
            present.setdefault(u, set()).add(w)
            if r0 == 0:
                first[u] = w
            if r1 == attended_len(stored[b], append_cap):
                last[u] = w
        if empty_unit is not None:
            slot = w + empty_unit
            assert slot not in slots and slot < N + units
            slots.add(slot)
            present.setdefault(empty_unit, set()).add(w)
    for b in range(B):
        L = attended_len(stored[b], append_cap)
        for ul in range(upb):
            u = b * upb + ul
            if not unit_rows(L, max_len, nq):
                assert u not in covered
                continue
            spans = sorted(covered[u])
            assert spans[0][0] == 0 and spans[-1][1] == L
            assert all(spans[i][1] == spans[i + 1][0] for i in range(len(spans) - 1)), spans
            assert present[u] == set(range(first[u], last[u] + 1))


@pytest.mark.parametrize("seed", range(8))
def test_partition_covers_every_row_once_with_distinct_slots(seed):
    rng = random.Random(1000 + seed)
    for _ in range(60):
        check_case(*draw_case(rng))


def test_shares_of_no_rows_inside_a_unit_leave_an_empty_partial():
    # 3 rows over 8 workgroups: some shares are empty and lie strictly inside the unit
    stored, upb, N = [3], 1, 8
    empties = [walk(w, N, stored, 10, 1, 0, upb, search_binary)[1] for w in range(N)]
    assert any(e == 0 for e in empties)
    check_case(stored, 10, 1, 0, upb, N)


def test_lanes_search_skips_sequences_without_rows():
    # prefixes [0, 5, 5, 5, 9]: a share starting at row 5 belongs to sequence 3
    pre = [0, 5, 5, 5, 9]
    assert search_lanes(pre, 5) == search_binary(pre, 5) == 3
    assert search_lanes(pre, 4) == search_binary(pre, 4) == 0
