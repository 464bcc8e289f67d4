"""Pins for oracle.routing: library stable sort, counting identities, edge cases."""

import numpy as np

from oracle.routing import route_buckets


def _check_valid(idx, E, counts, offsets, perm, slot):
    flat = idx.reshape(-1)
    routed = (flat >= 0) & (flat < E)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert offsets[-1] == routed.sum() == len(perm)
    assert sorted(perm.tolist()) == np.nonzero(routed)[0].tolist()
    assert np.all(np.diff(flat[perm]) >= 0)
    same = np.diff(flat[perm]) == 0
    assert np.all(np.diff(perm)[same] > 0)            # stable within an expert
    assert np.array_equal(slot[perm], np.arange(len(perm)))
    assert np.all(slot[~routed] == -1)


def test_matches_library_stable_argsort_and_bincount():
    rng = np.random.default_rng(31)
    for T, K, E in [(64, 2, 8), (333, 8, 64), (1000, 8, 128), (17, 4, 32)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, slot = route_buckets(idx, E)
        assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))
        assert np.array_equal(perm, np.argsort(idx.reshape(-1), kind="stable"))
        _check_valid(idx, E, counts, offsets, perm, slot)


def test_tiny_hand_case():
    idx = np.array([[2, 0], [0, 2], [1, 2]], np.int32)     # a = 0..5 -> experts 2,0,0,2,1,2
    counts, offsets, perm, slot = route_buckets(idx, 3)
    assert counts.tolist() == [2, 1, 3]
    assert offsets.tolist() == [0, 2, 3, 6]
    assert perm.tolist() == [1, 2, 4, 0, 3, 5]
    assert slot.tolist() == [3, 0, 1, 4, 2, 5]


def test_duplicates_empty_experts_and_out_of_range():
    idx = np.array([[3, 3], [3, -1], [9, 0]], np.int32)    # E = 4: -1 and 9 are not routed
    counts, offsets, perm, slot = route_buckets(idx, 4)
    assert counts.tolist() == [1, 0, 0, 3]
    assert offsets.tolist() == [0, 1, 1, 1, 4]
    assert perm.tolist() == [5, 0, 1, 2]
    assert slot.tolist() == [1, 2, 3, -1, -1, 0]
    _check_valid(idx, 4, counts, offsets, perm, slot)


def test_empty_input():
    counts, offsets, perm, slot = route_buckets(np.zeros((0, 2), np.int32), 5)
    assert counts.tolist() == [0] * 5 and offsets.tolist() == [0] * 6
    assert len(perm) == 0 and len(slot) == 0
