"""Pins for the oracle's stable token-to-expert grouping: brute force with
Python's sorted() on small random routings (including dropped ids, empty
experts, everything on one expert, zero rows) and structural invariants."""

import numpy as np
import pytest

from oracle import route_sort


def _brute(ids, E, tile_m):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    P = len(flat)
    valid = [p for p in range(P) if 0 <= flat[p] < E]
    order = sorted(valid, key=lambda p: (flat[p], p))
    dropped = [p for p in range(P) if not 0 <= flat[p] < E]
    counts = [sum(1 for p in valid if flat[p] == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    tiles = []
    for e in range(E):
        m0 = 0
        while m0 < counts[e]:
            tiles.append((e, offsets[e] + m0))
            m0 += tile_m
    return offsets, order + dropped, tiles


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("tile_m", [1, 3, 32, 256])
def test_matches_brute_force(seed, tile_m):
    g = np.random.default_rng(seed)
    E = int(g.integers(1, 12))
    rows = int(g.integers(0, 40))
    topk = int(g.integers(1, 5))
    ids = g.integers(-2, E + 2, (rows, topk)).astype(np.int32)
    off, sp, tiles = route_sort(ids, E, tile_m)
    b_off, b_sp, b_tiles = _brute(ids, E, tile_m)
    assert off.tolist() == b_off
    assert sp.tolist() == b_sp
    assert [tuple(t) for t in tiles.tolist()] == b_tiles


def test_invariants_and_degenerate_cases():
    E = 8
    ids = np.full((50, 2), 3, dtype=np.int32)                        # all to one expert
    off, sp, tiles = route_sort(ids, E, 16)
    assert off.tolist() == [0, 0, 0, 0, 100, 100, 100, 100, 100]
    assert sp.tolist() == list(range(100))
    assert tiles.tolist() == [[3, 0], [3, 16], [3, 32], [3, 48], [3, 64], [3, 80], [3, 96]]
    off, sp, tiles = route_sort(np.zeros((0, 4), dtype=np.int32), E, 16)
    assert off.tolist() == [0] * (E + 1) and sp.size == 0 and tiles.shape == (0, 2)
    g = np.random.default_rng(0)
    ids = g.integers(0, E, (300, 4)).astype(np.int32)
    off, sp, tiles = route_sort(ids, E, 32)
    assert sorted(sp.tolist()) == list(range(1200))
    assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=E))
    flat = ids.reshape(-1)
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_planted_swap_is_caught():
    """Positive control: swapping two entries of the oracle's answer breaks
    the brute-force comparison."""
    g = np.random.default_rng(1)
    ids = g.integers(0, 4, (20, 2)).astype(np.int32)
    off, sp, tiles = route_sort(ids, 4, 8)
    bad = sp.copy()
    bad[[0, 1]] = bad[[1, 0]]
    assert bad.tolist() != _brute(ids, 4, 8)[1]
