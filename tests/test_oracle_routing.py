"""Pins of the oracle's routing against a brute force built differently
(per-expert filtering instead of one counting pass) and against the
invariants any correct stable routing must satisfy; the tile-list checker
accepts two different valid tilings and rejects each kind of broken list."""
import numpy as np
import pytest

from oracle.routing import check_tiles, route


def brute_force(ids, E, row_pad, tile_rows):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    per_expert = [[p for p, v in enumerate(flat) if v == e] for e in range(E)]
    rows, pos, tiles = [], [-1] * len(flat), []
    for e, pairs in enumerate(per_expert):
        start = len(rows)
        for p in pairs:
            pos[p] = len(rows)
            rows.append(p)
        while len(rows) % row_pad:
            rows.append(-1)
        # fewest tiles of <= tile_rows rows, block counts differing by at most one, larger first
        blocks = (len(rows) - start) // row_pad
        if blocks:
            n = -(-blocks // (tile_rows // row_pad))   # whole blocks per tile
            sizes = sorted([blocks // n + (1 if i < blocks % n else 0) for i in range(n)], reverse=True)
            assert max(sizes) * row_pad <= tile_rows and max(sizes) - min(sizes) <= 1
            r = start
            for b in sizes:
                tiles.append((e, r, b * row_pad))
                r += b * row_pad
    counts = [len(p) for p in per_expert]
    return counts, rows, pos, tiles


CASES = [
    ("uniform", 16, 2, 8),
    ("one_hot_expert", 20, 4, 8),
    ("duplicates", 12, 3, 5),
    ("bad_ids", 10, 4, 6),
    ("empty", 0, 4, 8),
    ("many_experts_few_tokens", 3, 8, 128),
]


def _ids(kind, T, k, E, rng):
    if kind == "uniform" or kind == "many_experts_few_tokens":
        return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)
    if kind == "one_hot_expert":
        return np.full((T, k), 3, dtype=np.int32)
    if kind == "duplicates":
        return rng.integers(0, 2, size=(T, k)).astype(np.int32)
    if kind == "bad_ids":
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        ids[0, 0], ids[1, 1], ids[2, 2], ids[3, 3] = -1, E, 1000, -(2 ** 31)
        return ids
    return np.zeros((T, k), dtype=np.int32)


@pytest.mark.parametrize("kind,T,k,E", CASES)
@pytest.mark.parametrize("row_pad,tile_rows", [(1, 4), (16, 32), (16, 16), (4, 128), (16, 144), (2, 7)])
def test_route_matches_brute_force(kind, T, k, E, row_pad, tile_rows):
    rng = np.random.default_rng([sum(map(ord, kind)), row_pad, T, k])
    ids = _ids(kind, T, k, E, rng)
    r = route(ids, E, row_pad, tile_rows)
    counts, rows, pos, tiles = brute_force(ids, E, row_pad, tile_rows)
    assert r.counts.tolist() == counts
    assert r.sorted_ids.tolist() == rows
    assert r.pos.tolist() == pos
    assert r.offsets.tolist() == [0] + list(np.cumsum(counts))
    # two different valid tilings: the oracle's greedy one and the brute force's balanced one
    eff = tile_rows // row_pad * row_pad
    assert check_tiles(r.tiles, len(r.tiles), r.padded_offsets, E, row_pad, eff) == []
    assert check_tiles(np.array(tiles).reshape(-1, 3), len(tiles), r.padded_offsets, E, row_pad, eff) == []


@pytest.mark.parametrize("seed", range(5))
def test_route_invariants(seed):
    rng = np.random.default_rng(seed)
    E, T, k = 13, 37, 3
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    r = route(ids, E, 8, 24)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert r.counts.sum() == valid.sum()
    live = r.sorted_ids[r.sorted_ids >= 0]
    assert sorted(live.tolist()) == np.nonzero(valid)[0].tolist()      # a permutation of the valid pairs
    for i, p in enumerate(r.sorted_ids):
        if p >= 0:
            assert r.pos[p] == i and flat[p] == np.searchsorted(r.padded_offsets, i, side="right") - 1
    assert np.all(r.pos[~valid] == -1)
    assert np.all(np.diff(r.padded_offsets) % 8 == 0)
    for e in range(E):                                                 # stable: ascending p in each expert
        seg = r.sorted_ids[r.padded_offsets[e]:r.padded_offsets[e + 1]]
        seg = seg[seg >= 0]
        assert np.all(np.diff(seg) > 0)
    assert r.tiles[:, 2].sum() == r.padded_offsets[-1] and np.all(r.tiles[:, 2] <= 24)
    assert np.all(r.tiles[:, 2] % 8 == 0)


def test_check_tiles_rejects_broken_lists():
    ids = np.array([[0, 2], [2, 0], [2, 2], [0, 0], [2, 2]], dtype=np.int32)
    ids = np.concatenate([ids] * 7)                     # expert 0: 14 pairs, expert 2: 21, expert 1: none
    r = route(ids, 3, 4, 8)
    po = r.padded_offsets
    good = r.tiles.tolist()
    assert check_tiles(good, len(good), po, 3, 4, 8) == []
    assert check_tiles(good, len(good) + 1, po, 3, 4, 8)                    # wrong count
    bad = [list(t) for t in good]
    bad[1][1] += 4                                                           # a gap
    assert check_tiles(bad, len(bad), po, 3, 4, 8)
    bad = [list(t) for t in good]
    bad[0][2] += 4                                                           # too many rows / overlap
    assert check_tiles(bad, len(bad), po, 3, 4, 8)
    bad = [list(t) for t in good]
    bad[-1][2] = 2                                                           # not a multiple of row_pad
    assert check_tiles(bad, len(bad), po, 3, 4, 8)
    assert check_tiles(good[::-1], len(good), po, 3, 4, 8)                  # experts descending
    assert check_tiles(good[:-1], len(good) - 1, po, 3, 4, 8)               # last rows uncovered
    assert check_tiles(good + [[1, int(po[1]), 4]], len(good) + 1, po, 3, 4, 8)   # tile for an empty expert
    split = []
    for e, r0, n in good:                                                    # a finer valid tiling
        for k in range(0, n, 4):
            split.append([e, r0 + k, 4])
    assert check_tiles(split, len(split), po, 3, 4, 8) == []
