"""The balanced split-KV work partition (num_splits == 0 on the MFMA shapes),
checked as arithmetic on the CPU: the scheme the kernels implement is

  T tiles of all query rows, concatenated in row order, G = min(grid, ceil(T / 4))
  workgroups (at least 4 tiles each, at most one per compute unit); workgroup i takes tiles [i T / G, (i+1) T / G); the piece of
  row r inside it writes partial slot i + r; row r's partials are the slots
  g(first tile of r) + r .. g(last tile of r) + r with
  g(t) = ceil((t + 1) G / T) - 1 the workgroup holding tile t.

These tests restate that scheme and check its claims: every tile is covered
exactly once, slots are unique and fewer than grid + R (the workspace size),
and the slot range the combine reads for a row holds exactly that row's
pieces.  The GPU tests check the kernels against the oracle on such batches.
"""

from __future__ import annotations

import random


def pieces(tiles, grid):
    T = sum(tiles)
    G = min(grid, (T + 3) // 4)
    rs = [0]
    for t in tiles:
        rs.append(rs[-1] + t)
    out = {}
    for i in range(G):
        a, b = i * T // G, (i + 1) * T // G
        assert a < b, "no empty range"
        for r in range(len(tiles)):
            lo, hi = max(a, rs[r]) - rs[r], min(b, rs[r + 1]) - rs[r]
            if hi > lo:
                slot = i + r
                assert slot not in out, "slot used twice"
                out[slot] = (r, lo, hi)
    return out, rs, T, G


def combine_range(tiles, rs, T, G, r):
    if tiles[r] == 0:
        return range(0)
    g = lambda t: ((t + 1) * G + T - 1) // T - 1
    return range(g(rs[r]) + r, g(rs[r] + tiles[r] - 1) + r + 1)


def check(tiles, grid):
    if sum(tiles) == 0:
        return
    out, rs, T, G = pieces(tiles, grid)
    assert max(out) + 1 <= grid + len(tiles)
    for r in range(len(tiles)):
        slots = list(combine_range(tiles, rs, T, G, r))
        assert all(out[s][0] == r for s in slots)
        covered = sorted(t for s in slots for t in range(out[s][1], out[s][2]))
        assert covered == list(range(tiles[r]))
    assert sorted(out) == sorted(s for r in range(len(tiles))
                                 for s in combine_range(tiles, rs, T, G, r))


def test_uniform_batch_matches_four_splits_per_row():
    # 64 rows x 128 tiles on 256 workgroups: 32 tiles each, 4 per row
    out, _, _, _ = pieces([128] * 64, 256)
    assert len(out) == 256
    assert all(hi - lo == 32 for (_, lo, hi) in out.values())


def test_fewer_tiles_than_workgroups():
    check([1, 2], 256)
    check([0, 3, 0], 256)


def test_random_ragged_batches():
    rng = random.Random(1)
    for _ in range(400):
        R = rng.randint(1, 200)
        grid = rng.choice([1, 7, 64, 256])
        tiles = [rng.choice([0, 1, 2, 3, rng.randint(0, 600)]) for _ in range(R)]
        check(tiles, grid)
