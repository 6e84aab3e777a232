"""Pins for the oracle's affinity-based token dropping: brute force over the
kept sets on tiny inputs, and the cases that reduce to no dropping or to
dropping everything."""
import itertools

import numpy as np
import pytest

from oracle import moe_ref as ref


def _pairs(idx, g0, group):
    T, k = idx.shape
    return [(t, j) for t in range(T) for j in range(k) if g0 <= idx[t, j] < g0 + group]


@pytest.mark.parametrize("seed,E,k,group,cap", [(0, 4, 2, 1, 2), (1, 6, 2, 2, 3), (2, 4, 1, 4, 3),
                                                (3, 8, 3, 2, 4)])
def test_capacity_drop_keeps_the_highest_affinities(seed, E, k, group, cap):
    rng = np.random.default_rng(seed)
    T = 7
    L = rng.standard_normal((T, E))
    idx, _ = ref.topk_softmax(L, k)
    out = ref.capacity_drop(idx, L, E, group, cap)
    # brute force: softmax by hand, every subset of size cap of each group
    s = np.exp(L) / np.exp(L).sum(axis=1, keepdims=True)
    for g0 in range(0, E, group):
        pairs = _pairs(idx, g0, group)
        kept = [p for p in pairs if out[p] >= 0]
        assert len(kept) == min(cap, len(pairs))
        best = max(itertools.combinations(pairs, min(cap, len(pairs))),
                   key=lambda c: sum(s[t, idx[t, j]] for t, j in c))
        assert sorted(kept) == sorted(best)
        for t, j in kept:
            assert out[t, j] == idx[t, j]          # kept ids unchanged


def test_capacity_ties_follow_dispatch_order():
    T, E = 6, 2
    L = np.zeros((T, E))                          # every affinity is 1/2
    idx = np.zeros((T, 1), int)
    idx[3:] = 1
    out = ref.capacity_drop(idx, L, E, 2, 4)      # one group of both experts
    np.testing.assert_array_equal(out.ravel(), [0, 0, 0, 1, -1, -1])


def test_capacity_limits():
    rng = np.random.default_rng(5)
    T, E, k = 20, 4, 2
    L = rng.standard_normal((T, E))
    idx, _ = ref.topk_softmax(L, k)
    np.testing.assert_array_equal(ref.capacity_drop(idx, L, E, 1, T), idx)   # never full
    assert (ref.capacity_drop(idx, L, E, 2, 0) == -1).all()                  # nothing kept
    np.testing.assert_array_equal(ref.capacity_drop(idx, L, E, E, T * k), idx)
