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
