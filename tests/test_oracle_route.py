"""Pins for oracle.route: brute force against Python's stable sorted() and the
permutation invariants."""
import numpy as np

from oracle.route import route


def brute(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    valid = [r for r, e in enumerate(flat) if 0 <= e < E]
    srt = sorted(valid, key=lambda r: (flat[r], r))
    counts = [sum(1 for r in valid if flat[r] == e) for e in range(E)]
    return counts, srt


def test_route_brute_force_with_masks_and_duplicates():
    rng = np.random.default_rng(0)
    for trial in range(40):
        T, k, E = int(rng.integers(0, 40)), int(rng.integers(1, 7)), int(rng.integers(1, 20))
        ids = rng.integers(-2, E + 2, (T, k))            # some ids out of range, duplicates allowed
        counts, offsets, srt, pos = route(ids, E)
        bc, bs = brute(ids, E)
        assert list(counts) == bc
        assert list(srt) == bs
        assert offsets[0] == 0 and np.all(np.diff(offsets) == counts)
        assert offsets[-1] == len(bs)
        flat = ids.reshape(-1)
        for r in range(T * k):
            if 0 <= flat[r] < E:
                assert srt[pos[r]] == r
                assert offsets[flat[r]] <= pos[r] < offsets[flat[r] + 1]
            else:
                assert pos[r] == -1


def test_route_empty_and_single_expert():
    counts, offsets, srt, pos = route(np.zeros((0, 3), np.int32), 4)
    assert list(counts) == [0] * 4 and list(offsets) == [0] * 5 and srt.size == 0 and pos.size == 0
    ids = np.full((5, 2), 3)
    counts, offsets, srt, pos = route(ids, 4)
    assert list(counts) == [0, 0, 0, 10] and list(srt) == list(range(10)) and list(pos) == list(range(10))
