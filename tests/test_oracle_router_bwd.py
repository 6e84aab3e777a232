"""Pins for the oracle's router backward and load-balance loss.

The loss is  sum_t <dy_t, y_t> + L_aux  with the top-k selection held fixed
(it is piecewise constant in the logits): central finite differences in fp64
and torch CPU autograd of the same function, closed forms of L_aux, and the
shift invariance of a softmax (every token's logit gradient sums to zero).
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as ref


def _setup(seed, T=7, h=6, hf=5, E=4, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h))
    wg = rng.standard_normal((h, E)) * 0.7
    b = rng.standard_normal(E) * 0.3
    w1 = rng.standard_normal((E, h, hf)) * 0.6
    w3 = rng.standard_normal((E, h, hf)) * 0.6
    w2 = rng.standard_normal((E, hf, h)) * 0.6
    dy = rng.standard_normal((T, h))
    idx, _ = ref.topk_softmax(ref.router_logits(x, wg, b).astype(np.float64), k)
    return x, wg, b, w1, w3, w2, dy, idx


def _loss(x, wg, b, w1, w3, w2, dy, idx, alpha):
    """sum_t <dy_t, y_t> + L_aux with routing idx fixed (fp64 throughout)."""
    L = x @ wg + b
    sel = np.take_along_axis(L, idx, axis=1)
    w = ref.softmax_rows(sel)
    y = ref.layer_forward_tokens(x, idx, w, w1, w3, w2)
    return float(np.sum(dy * y)) + ref.aux_balance_loss(L, idx, wg.shape[1], idx.shape[1], alpha)


def _grads(x, wg, b, w1, w3, w2, dy, idx, alpha):
    L = x @ wg + b
    w = ref.softmax_rows(np.take_along_axis(L, idx, axis=1))
    ysel = np.stack([np.stack([ref.layer_forward_tokens(x[t:t + 1], idx[t:t + 1, j:j + 1],
                                                       np.ones((1, 1)), w1, w3, w2)[0]
                               for j in range(idx.shape[1])]) for t in range(x.shape[0])])
    rb = ref.router_backward(dy, ysel, x, wg, L, idx, w, alpha)
    dx_expert = ref.layer_backward_tokens(dy, x, idx, w, w1, w3, w2)
    return rb, dx_expert


def _fd(f, a, eps=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        p, m = a.copy(), a.copy()
        p[i] += eps
        m[i] -= eps
        g[i] = (f(p) - f(m)) / (2 * eps)
    return g


@pytest.mark.parametrize("seed,alpha,k", [(0, 0.0, 2), (1, 0.3, 2), (2, 0.7, 3), (3, 0.5, 1)])
def test_router_backward_matches_finite_differences(seed, alpha, k):
    x, wg, b, w1, w3, w2, dy, idx = _setup(seed, k=k)
    rb, dx_expert = _grads(x, wg, b, w1, w3, w2, dy, idx, alpha)
    f = lambda **kw: _loss(kw.get("x", x), kw.get("wg", wg), kw.get("b", b), w1, w3, w2, dy, idx, alpha)
    for name, arr, got in (("wg", wg, rb["dw_gate"]), ("b", b, rb["dbias"]), ("x", x, rb["dx"] + dx_expert)):
        num = _fd(lambda a: f(**{name: a}), arr)
        scale = np.abs(num).max()
        assert scale > 0
        assert np.abs(num - got).max() <= 1e-6 * scale, name


def test_router_backward_matches_torch_autograd():
    x, wg, b, w1, w3, w2, dy, idx = _setup(5, T=9, h=6, hf=7, E=5, k=3)
    alpha = 0.4
    rb, dx_expert = _grads(x, wg, b, w1, w3, w2, dy, idx, alpha)
    tx, tg, tb = (torch.tensor(a, requires_grad=True) for a in (x, wg, b))
    T, E, k = x.shape[0], wg.shape[1], idx.shape[1]
    ti = torch.tensor(idx.astype(np.int64))
    L = tx @ tg + tb
    w = torch.softmax(torch.gather(L, 1, ti), dim=1)
    y = torch.zeros_like(tx)
    W1, W3, W2 = (torch.tensor(a) for a in (w1, w3, w2))
    for j in range(k):
        e = ti[:, j]
        g = torch.einsum("th,thf->tf", tx, W1[e])
        u = torch.einsum("th,thf->tf", tx, W3[e])
        y = y + w[:, j:j + 1] * torch.einsum("tf,tfh->th", torch.nn.functional.silu(g) * u, W2[e])
    counts = torch.bincount(ti.reshape(-1), minlength=E).to(torch.float64)
    aux = alpha * torch.sum(E / (k * T) * counts * torch.softmax(L, dim=1).mean(dim=0))
    ((y * torch.tensor(dy)).sum() + aux).backward()
    np.testing.assert_allclose(rb["dw_gate"], tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rb["dbias"], tb.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rb["dx"] + dx_expert, tx.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_logit_gradient_rows_sum_to_zero():
    # adding a constant to all of a token's logits changes neither softmax
    x, wg, b, w1, w3, w2, dy, idx = _setup(7, T=11, E=6, k=2)
    rb, _ = _grads(x, wg, b, w1, w3, w2, dy, idx, 0.8)
    assert np.abs(rb["dL"].sum(axis=1)).max() < 1e-12 * np.abs(rb["dL"]).max()


def test_top1_gate_has_no_logit_gradient_without_aux():
    # k = 1: the single gate weight is exactly 1 whatever the logits
    x, wg, b, w1, w3, w2, dy, idx = _setup(8, k=1)
    rb, _ = _grads(x, wg, b, w1, w3, w2, dy, idx, 0.0)
    assert not rb["dL"].any()
    assert not rb["dw_gate"].any()


def test_aux_loss_closed_forms():
    T, E, k, alpha = 12, 4, 2, 0.25
    # equal logits and exactly balanced routing: f_e = 1, P_e = 1/E -> alpha
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    assert ref.aux_balance_loss(np.zeros((T, E)), idx, E, k, alpha) == pytest.approx(alpha, rel=1e-15)
    # every token on expert 0 (k = 1): f_0 = E, loss = alpha * E * mean_t softmax(L_t)_0
    rng = np.random.default_rng(0)
    L = rng.standard_normal((T, E))
    p0 = np.mean([np.exp(L[t, 0]) / np.exp(L[t]).sum() for t in range(T)])
    assert ref.aux_balance_loss(L, np.zeros((T, 1), int), E, 1, alpha) == pytest.approx(alpha * E * p0, rel=1e-13)


def test_aux_gradient_alone_matches_finite_differences():
    rng = np.random.default_rng(4)
    T, E, k, alpha = 10, 6, 2, 1.3
    L = rng.standard_normal((T, E))
    idx, _ = ref.topk_softmax(L, k)
    rb = ref.router_backward(np.zeros((T, 3)), np.zeros((T, k, 3)), np.zeros((T, 3)), np.zeros((3, E)),
                             L, idx, np.full((T, k), 1.0 / k), alpha)
    num = _fd(lambda a: ref.aux_balance_loss(a, idx, E, k, alpha), L)
    assert np.abs(num - rb["dL"]).max() <= 1e-8 * np.abs(num).max()


def test_bf16_storage_forward_rounds_a_only():
    rng = np.random.default_rng(11)
    E, h, hf, R = 3, 8, 6, 20
    xp = ref.round_bf16(rng.standard_normal((R, h)))
    offs = np.array([0, 7, 7, 20])
    w1, w3 = rng.standard_normal((E, h, hf)), rng.standard_normal((E, h, hf))
    w2 = rng.standard_normal((E, hf, h))
    ex, _, _, a = ref.expert_forward(xp, offs, w1, w3, w2)
    st, _, _, a_st = ref.expert_forward(xp, offs, w1, w3, w2, bf16_storage=True)
    np.testing.assert_array_equal(a_st, ref.round_bf16(a))         # A rounded once
    for e in range(E):                                             # FC2 from the rounded A, not rounded
        lo, hi = offs[e], offs[e + 1]
        np.testing.assert_array_equal(st[lo:hi], ref.round_bf16(a[lo:hi]) @ w2[e])
    rel = np.abs(st - ex).max() / np.abs(ex).max()
    assert 0 < rel < 2e-2


def test_router_backward_on_a_subset_of_tokens():
    """Rows of a subset, given the batch's counts and token count, equal the
    same rows of the whole batch's evaluation (the balance-loss term depends
    on the batch only through those two)."""
    x, wg, b, w1, w3, w2, dy, idx = _setup(11, T=13, E=5, k=2)
    L = x @ wg + b
    w = ref.softmax_rows(np.take_along_axis(L, idx, axis=1))
    ysel = np.stack([np.stack([ref.layer_forward_tokens(x[t:t + 1], idx[t:t + 1, j:j + 1],
                                                       np.ones((1, 1)), w1, w3, w2)[0]
                               for j in range(idx.shape[1])]) for t in range(x.shape[0])])
    full = ref.router_backward(dy, ysel, x, wg, L, idx, w, 0.6)
    sub = np.array([1, 4, 5, 11])
    counts = np.bincount(idx.ravel(), minlength=wg.shape[1])
    part = ref.router_backward(dy[sub], ysel[sub], x[sub], wg, L[sub], idx[sub], w[sub], 0.6, counts=counts,
                               T_batch=x.shape[0])
    np.testing.assert_allclose(part["dL"], full["dL"][sub], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part["dx"], full["dx"][sub], rtol=1e-13, atol=1e-15)
