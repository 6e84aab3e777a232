"""Pins for the oracle's index builder and the dispatch / combine copies.

Pins: ``np.bincount`` for the histogram, a stable ``np.argsort`` of the
flattened expert ids for the permutation (a library routine that must agree
with the expert-then-token order), and the invariants "counts sum to T*k" and
"un-permute after permute is the identity".
"""
import numpy as np
import pytest

from oracle import moe_ref as ref


def _route(T, E, k, seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    return ref.topk_softmax(L, k)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (13, 4, 2), (256, 8, 2), (300, 64, 6), (50, 16, 1)])
def test_index_matches_stable_argsort(T, E, k):
    idx, _ = _route(T, E, k, T + E)
    counts, offsets, dst_row, src_tok = ref.build_index(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[E] == T * k
    np.testing.assert_array_equal(np.diff(offsets), counts)
    order = np.argsort(idx.ravel(), kind="stable")          # entry id placed at each row
    np.testing.assert_array_equal(dst_row.ravel()[order], np.arange(T * k))
    np.testing.assert_array_equal(src_tok, order // k)
    # rows of one expert are contiguous and their tokens ascend
    for e in range(E):
        toks = src_tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)


def test_empty_and_degenerate():
    counts, offsets, dst_row, src_tok = ref.build_index(np.zeros((0, 2), np.int32), 4)
    assert counts.tolist() == [0, 0, 0, 0] and offsets.tolist() == [0] * 5
    assert dst_row.shape == (0, 2) and src_tok.shape == (0,)
    idx = np.zeros((10, 1), np.int32) + 3                     # everyone to expert 3
    counts, offsets, dst_row, src_tok = ref.build_index(idx, 5)
    assert counts.tolist() == [0, 0, 0, 10, 0]
    np.testing.assert_array_equal(dst_row[:, 0], np.arange(10))


def test_permute_unpermute_identity():
    T, E, k, h = 40, 8, 3, 5
    idx, w = _route(T, E, k, 3)
    _, _, dst_row, src_tok = ref.build_index(idx, E)
    x = np.random.default_rng(0).standard_normal((T, h)).astype(np.float32)
    xp = ref.permute(x, dst_row)
    for j in range(k):
        np.testing.assert_array_equal(xp[dst_row[:, j]], x)
    np.testing.assert_array_equal(xp, x[src_tok])
    # combine with unit weights sums the k copies
    np.testing.assert_allclose(ref.combine(xp, dst_row, None), k * x.astype(np.float64), rtol=1e-15)


def test_identity_experts_return_x():
    """Combine with identity experts equals the gate-weighted sum of x, i.e. x."""
    T, E, k, h = 64, 8, 2, 16
    idx, w = _route(T, E, k, 11)
    _, _, dst_row, _ = ref.build_index(idx, E)
    x = np.random.default_rng(2).standard_normal((T, h)).astype(np.float32)
    y = ref.combine(ref.permute(x, dst_row), dst_row, w)
    np.testing.assert_allclose(y, x, rtol=0, atol=4e-7 * np.abs(x).max())
    np.testing.assert_allclose(y, w.astype(np.float64).sum(1)[:, None] * x, rtol=1e-15)


def test_row_scaled_permute():
    T, E, k, h = 20, 4, 2, 3
    idx, w = _route(T, E, k, 4)
    _, _, dst_row, _ = ref.build_index(idx, E)
    x = np.random.default_rng(3).standard_normal((T, h))
    xp = ref.permute(x, dst_row, row_scale=w)
    for t in range(T):
        for j in range(k):
            np.testing.assert_allclose(xp[dst_row[t, j]], w[t, j] * x[t], rtol=1e-15)


def test_build_index_drops_ids_outside_range():
    idx = np.array([[0, 3], [-1, 1], [2, 7], [1, 0]])
    counts, offsets, dst_row, src_tok = ref.build_index(idx, 4)
    np.testing.assert_array_equal(counts, [2, 2, 1, 1])
    np.testing.assert_array_equal(offsets, [0, 2, 4, 5, 6])
    np.testing.assert_array_equal(dst_row, [[0, 5], [-1, 2], [4, -1], [3, 1]])
    np.testing.assert_array_equal(src_tok, [0, 3, 1, 3, 2, 0, -1, -1])


def test_expert_parallel_shares_partition_the_layer():
    """n GPUs' shares (expert ranges) together route every pair exactly once,
    and their partial combines add up to the full combine."""
    rng = np.random.default_rng(3)
    T, E, k, h, n = 40, 8, 3, 5, 4
    L = rng.standard_normal((T, E))
    idx, w = ref.topk_softmax(L, k)
    counts, offsets, dst_row, _ = ref.build_index(idx, E)
    yp = rng.standard_normal((T * k, h))
    full = ref.combine(yp, dst_row, w)
    total = np.zeros_like(full)
    seen = np.zeros((T, k), int)
    for r in range(n):
        e_lo = r * E // n
        loc = ref.local_expert_ids(idx, e_lo, E // n)
        c_r, o_r, d_r, s_r = ref.build_index(loc, E // n)
        np.testing.assert_array_equal(c_r, counts[e_lo:e_lo + E // n])   # a slice of the global counts
        seen += d_r >= 0
        # the rank's rows, in its own order, carry the same expert outputs
        yp_r = np.zeros((max(int(o_r[-1]), 1), h))
        yp_r[d_r[d_r >= 0]] = yp[dst_row[d_r >= 0]]
        total += ref.combine(yp_r, d_r, w)
        # rows of each local expert are ordered by token (= by source rank,
        # when ranks own contiguous token ranges)
        for e in range(E // n):
            toks = s_r[o_r[e]:o_r[e + 1]]
            assert np.all(np.diff(toks) > 0)
    assert np.all(seen == 1)
    np.testing.assert_allclose(total, full, rtol=1e-13, atol=1e-13)


def test_index_with_repeated_ids_in_a_token():
    """A token naming one expert in several slots: every (token, slot) pair
    is its own row, the token's pairs consecutive and in slot order (the
    stable argsort of the flattened ids), and un-permute after permute still
    returns each pair's token."""
    rng = np.random.default_rng(17)
    T, E, k = 300, 6, 4
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)    # repeats in most tokens
    idx[5] = 2                                                # all four slots on one expert
    counts, offsets, dst_row, src_tok = ref.build_index(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    order = np.argsort(idx.ravel(), kind="stable")
    np.testing.assert_array_equal(dst_row.ravel()[order], np.arange(T * k))
    np.testing.assert_array_equal(src_tok, order // k)
    assert np.all(np.diff(dst_row[5]) == 1)
    assert len(np.unique(dst_row)) == T * k
