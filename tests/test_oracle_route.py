"""Pins for the oracle's routing: gate GEMM, top-k order and softmax weights.

Pins used: exact integer arithmetic for the gate product, a per-token
pure-Python brute force, the k = E special case against scipy's softmax, and
the invariants "k distinct experts", "weights sum to one", "weights
non-increasing", "k = 1 gives weight 1".
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe_ref as ref


def _brute_route(L, k):
    T, E = L.shape
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
        vals = [float(L[t, e]) for e in order]
        z = [math.exp(v - vals[0]) for v in vals]
        s = math.fsum(z)
        idx[t] = order
        w[t] = [zi / s for zi in z]
    return idx, w


def test_gate_gemm_exact_on_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 8, size=(7, 16)).astype(np.float32)
    wg = rng.integers(-8, 8, size=(16, 5)).astype(np.float32)
    b = np.array([0.5, -1.0, 0.0, 2.0, 0.25], np.float32)
    L = ref.router_logits(x, wg, b)
    want = np.zeros((7, 5))
    for t in range(7):
        for e in range(5):
            want[t, e] = sum(float(x[t, i]) * float(wg[i, e]) for i in range(16)) + float(b[e])
    assert L.dtype == np.float32
    np.testing.assert_array_equal(L, want.astype(np.float32))


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 8, 2), (33, 64, 6), (16, 16, 1), (9, 5, 5)])
def test_topk_matches_bruteforce(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = ref.topk_softmax(L, k)
    bi, bw = _brute_route(L, k)
    np.testing.assert_array_equal(idx, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-7, atol=0)


def test_ties_break_to_lower_index():
    L = np.array([[1.0, 3.0, 3.0, 1.0, 3.0],
                  [0.0, -0.0, 0.0, -1.0, 0.0],
                  [2.0, 2.0, 2.0, 2.0, 2.0]], np.float32)
    idx, w = ref.topk_softmax(L, 3)
    np.testing.assert_array_equal(idx, [[1, 2, 4], [0, 1, 2], [0, 1, 2]])
    np.testing.assert_allclose(w, np.full((3, 3), 1 / 3), rtol=1e-7)
    bi, _ = _brute_route(L, 3)
    np.testing.assert_array_equal(idx, bi)


def test_invariants():
    rng = np.random.default_rng(5)
    L = (rng.standard_normal((200, 16)) * 3).astype(np.float32)
    for k in (1, 2, 4, 16):
        idx, w = ref.topk_softmax(L, k)
        assert idx.dtype == np.int32 and w.dtype == np.float32
        for t in range(L.shape[0]):
            assert len(set(idx[t].tolist())) == k
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)
        assert np.all(np.diff(w, axis=1) <= 0)
        if k == 1:
            assert np.all(w == 1.0)


def test_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((50, 8)).astype(np.float32)
    idx, w = ref.topk_softmax(L, 8)
    full = softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, idx, 1), rtol=1e-6)


def test_margin():
    L = np.array([[3.0, 1.0, 2.0, 0.5]], np.float32)
    np.testing.assert_allclose(ref.topk_margin(L, 1), [1.0])
    np.testing.assert_allclose(ref.topk_margin(L, 2), [1.0])
    np.testing.assert_allclose(ref.topk_margin(L, 3), [0.5])
    assert np.isinf(ref.topk_margin(L, 4)[0])
