"""The balanced split-KV work partition (num_splits == 0 on the MFMA shapes),
checked as arithmetic on the CPU.  The scheme the kernels implement:

  Query row r = b q + s (q = q_len) sees L_b - q + s + 1 tokens, tiles(r) =
  ceil of that / 64.  The partition runs over entries: with 1 < q <= 8 an
  entry is a sequence (Qs = q rows; its tiles are its last row's), otherwise
  an entry is a row (Qs = 1).  The T entry tiles, concatenated in order, are
  cut into G = min(8 floor(grid / 8 / Qs), T) ranges [g T / G, (g+1) T / G).
  Range g is walked by Qs workgroups, row s each; the piece of (g, entry e,
  row s) writes partial slot Qs (g + e) + s, holding the range's tiles that
  row sees (none: log-sum-exp -inf).  The combine reads row (e, s)'s partials
  at slots Qs (f + e) + s .. Qs (l + e) + s, step Qs, f / l = the ranges
  holding the entry's first / last tile, grp(t) = ceil((t + 1) G / T) - 1.
  Workgroup id b (XCD b % 8) takes range (b % 8) ceil(G / 8) + (b / 8) / Qs
  and row (b / 8) % Qs when (b / 8) < Qs ceil(G / 8).

These tests restate that scheme and check its claims: every tile of every
row is covered exactly once, slots are unique and fewer than grid + R (the
workspace size), the combine's slots for a row hold exactly that row's
pieces, and the workgroups of one range sit on one XCD.  The GPU tests check
the kernels against the oracle on such batches.
"""

from __future__ import annotations

import random

PAIR_Q = 8
BS = 64


def row_tiles(lens, q, r):
    b, s = divmod(r, q)
    n = lens[b] - q + s + 1
    return (n + BS - 1) // BS if n > 0 else 0


def schedule(lens, q, grid):
    R = len(lens) * q
    Qs = q if q <= PAIR_Q else 1
    E = R // Qs

    def entry_row(e, s):
        return e * q + s if q <= PAIR_Q else e

    etiles = [row_tiles(lens, q, entry_row(e, Qs - 1)) for e in range(E)]
    es = [0]
    for t in etiles:
        es.append(es[-1] + t)
    T = es[-1]
    G = min(8 * ((grid // 8) // Qs), T)
    pieces = {}                   # slot -> (row, lo, hi); hi == lo: an empty piece (lse -inf)
    for g in range(G):
        a, b = g * T // G, (g + 1) * T // G
        assert a < b, "no empty range"
        for s in range(Qs):
            for e in range(E):
                lo, hi = max(a, es[e]) - es[e], min(b, es[e + 1]) - es[e]
                if hi > lo:
                    row = entry_row(e, s)
                    slot = Qs * (g + e) + s
                    assert slot not in pieces, "slot used twice"
                    pieces[slot] = (row, lo, max(lo, min(hi, row_tiles(lens, q, row))))
    return dict(pieces=pieces, es=es, etiles=etiles, T=T, G=G, Qs=Qs, E=E, R=R,
                entry_row=entry_row)


def combine_slots(sc, r):
    Qs, T, G = sc["Qs"], sc["T"], sc["G"]
    e, s = (r // Qs, r % Qs)
    n = sc["etiles"][e]
    if n == 0:
        return []
    grp = lambda t: ((t + 1) * G + T - 1) // T - 1
    f, l = grp(sc["es"][e]), grp(sc["es"][e] + n - 1)
    return [Qs * (g + e) + s for g in range(f, l + 1)]


def workgroup_units(G, Qs, grid):
    per = (G + 7) // 8
    units = {}
    for b in range(grid):
        bx, bk = b % 8, b // 8
        if bk < per * Qs:
            g = bx * per + bk // Qs
            if g < G:
                units[b] = (g, bk % Qs)
    return units


def check(lens, q, grid=256):
    sc = schedule(lens, q, grid)
    if sc["T"] == 0:
        return
    pieces, R = sc["pieces"], sc["R"]
    assert max(pieces) + 1 <= grid + R
    for r in range(R):
        slots = combine_slots(sc, r)
        assert all(s in pieces and pieces[s][0] == r for s in slots)
        covered = sorted(t for s in slots for t in range(pieces[s][1], pieces[s][2]))
        assert covered == list(range(row_tiles(lens, q, r)))
    assert sorted(pieces) == sorted(s for r in range(R) for s in combine_slots(sc, r))
    units = workgroup_units(sc["G"], sc["Qs"], grid)
    assert sorted(units.values()) == [(g, s) for g in range(sc["G"]) for s in range(sc["Qs"])]
    xcd = {}
    for b, (g, s) in units.items():
        assert xcd.setdefault(g, b % 8) == b % 8, "a range's rows on two XCDs"


def test_uniform_batch_matches_four_ranges_per_row():
    # 64 rows x 128 tiles on 256 workgroups: 32 tiles each, 4 per row
    sc = schedule([8192] * 64, 1, 256)
    assert len(sc["pieces"]) == 256
    assert all(hi - lo == 32 for (_, lo, hi) in sc["pieces"].values())


def test_one_tile_per_workgroup_for_a_short_row():
    # one 4096-token row: 64 tiles on 64 workgroups
    sc = schedule([4096], 1, 256)
    assert sc["G"] == 64 and len(sc["pieces"]) == 64


def test_two_query_rows_share_ranges():
    # 128 sequences x 2 rows: 128 ranges, each walked by two workgroups (one per
    # row) over the same tiles; slots 2 (g + e) + s
    lens = [8192 + 64 * i for i in range(128)]
    sc = schedule(lens, 2, 256)
    assert sc["Qs"] == 2 and sc["G"] == 128
    by_range = {}
    for slot, (row, lo, hi) in sc["pieces"].items():
        by_range.setdefault(slot // 2, []).append((row % 2, row // 2, lo, hi))
    for items in by_range.values():
        # both rows of a (range, sequence) piece cover the same tiles
        assert len({(e, lo) for (_, e, lo, _) in items}) == 1
    check(lens, 2)


def test_fewer_tiles_than_workgroups():
    check([1, 2], 1)
    check([0, 3, 0], 1)
    check([1, 2], 2)
    check([2, 1, 1, 70], 3)


def test_row_that_sees_nothing_gets_empty_pieces():
    # q_len 2, length 1: row 0 sees no token, row 1 sees one
    sc = schedule([1, 65], 2, 256)
    empty = [s for s, (row, lo, hi) in sc["pieces"].items() if hi == lo]
    assert empty and all(sc["pieces"][s][0] % 2 == 0 for s in empty)
    check([1, 65], 2)


def test_random_ragged_batches():
    rng = random.Random(1)
    for _ in range(300):
        q = rng.choice([1, 1, 2, 3, 4, 8, 9, 16])
        B = rng.randint(1, max(1, 200 // q))
        grid = rng.choice([64, 256])         # multiples of 8 with grid / 8 >= 8 rows per range
        lens = [rng.choice([0, 1, 2, 63, 64, 65, rng.randint(0, 40000)]) for _ in range(B)]
        check(lens, q, grid)
