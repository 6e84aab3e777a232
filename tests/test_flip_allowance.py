"""Pins for the one-operand-flip allowance of the BF16 backward comparison.

The allowance must (a) cover the change that one BF16 operand rounded to its
neighbouring value makes to the oracle's BF16-operand weight gradients, and
(b) not cover errors that move whole terms (a dropped row, swapped rows).
The flips are planted in the oracle on the CPU: its BF16 rounding is wrapped
so that one element of one operand goes to the neighbouring BF16 value.
"""
import numpy as np
import pytest

from oracle import moe_ref as ref
from bf16_flip import bf16_step, weight_grad_flip_allowance

_RB = ref.round_bf16  # the oracle's own rounding, kept before any wrapping


def test_bf16_step_is_the_spacing_of_bf16_values():
    for v, st in ((1.0, 2.0 ** -7), (1.5, 2.0 ** -7), (-3.0, 2.0 ** -6), (0.0, 0.0),
                  (2.0 ** -20 * 1.75, 2.0 ** -27), (300.0, 2.0)):
        assert bf16_step(v) == st, v
    rng = np.random.default_rng(0)
    v = ref.round_bf16(rng.standard_normal(1000) * np.exp(rng.uniform(-8, 8, 1000)))
    st = bf16_step(v)
    # the next BF16 value away from zero is exactly one step further, none lies between
    np.testing.assert_array_equal(ref.round_bf16(v + np.sign(v) * st), v + np.sign(v) * st)
    np.testing.assert_array_equal(ref.round_bf16(v + np.sign(v) * 0.49 * st), v)


def _case(seed, T=48, h=16, hf=12):
    """One expert, k = 1: the routed rows are the tokens in order, weight 1."""
    rng = np.random.default_rng(seed)
    x = ref.round_bf16(rng.standard_normal((T, h)))
    w1 = ref.round_bf16(rng.standard_normal((1, h, hf)) * 0.5)
    w3 = ref.round_bf16(rng.standard_normal((1, h, hf)) * 0.5)
    w2 = ref.round_bf16(rng.standard_normal((1, hf, h)) * 0.5)
    dy = ref.round_bf16(rng.standard_normal((T, h)))
    dst_row = np.arange(T).reshape(T, 1)
    offsets = np.array([0, T])
    w = np.ones((T, 1))
    return x, dy, w, dst_row, offsets, w1, w3, w2


def _grads(case, monkeypatch=None, call=None, edit=None):
    """expert_grads with BF16 operands; the call-th BF16 rounding (1: dYp, 2: G,
    3: U, 4: dG, 5: dU, 6: A) has ``edit`` applied to its result."""
    x, dy, w, dst_row, offsets, w1, w3, w2 = case
    if monkeypatch is not None:
        orig = _RB
        seen = [0]

        def rb(a):
            r = orig(a)
            seen[0] += 1
            return edit(r.copy()) if seen[0] == call else r
        monkeypatch.setattr(ref, "round_bf16", rb)
    out = ref.expert_grads(x, dy, w1[0], w3[0], w2[0], bf16_operands=True)
    if monkeypatch is not None:
        monkeypatch.undo()
    return dict(zip(("dw1", "dw3", "dw2"), out[:3]))


def test_expert_grads_equal_layer_backward_for_one_expert():
    case = _case(0)
    x, dy, w, dst_row, offsets, w1, w3, w2 = case
    lb = ref.layer_backward(dy, x, w, dst_row, offsets, w1, w3, w2, bf16_operands=True)
    eg = _grads(case)
    for name in eg:
        np.testing.assert_allclose(eg[name], lb[name][0], rtol=1e-12, atol=1e-12)


def _flip(r, n, sign):
    def edit(a):
        a[r, n] = _RB(np.array([a[r, n] + sign * bf16_step(a[r, n])]))[0]
        return a
    return edit


# operand -> the weight gradients the allowance covers for its flip
COVERED = {1: ("dw2",), 2: ("dw1", "dw3", "dw2"), 3: ("dw1", "dw2"), 4: ("dw1",), 5: ("dw3",), 6: ("dw2",)}


@pytest.mark.parametrize("call", sorted(COVERED))
@pytest.mark.parametrize("seed", [1, 2])
def test_one_planted_flip_is_within_the_allowance(monkeypatch, call, seed):
    case = _case(seed)
    x, dy, w, dst_row, offsets, w1, w3, w2 = case
    allow = weight_grad_flip_allowance(dy, x, w, dst_row, offsets, w1, w3, w2)
    base = _grads(case)
    rng = np.random.default_rng(100 + seed)
    moved = 0.0
    for _ in range(6):
        cols = x.shape[1] if call == 1 else w1.shape[2]
        r, n, sign = int(rng.integers(0, x.shape[0])), int(rng.integers(0, cols)), float(rng.choice([-1, 1]))
        got = _grads(case, monkeypatch, call, _flip(r, n, sign))
        for name in COVERED[call]:
            d = np.abs(got[name] - base[name])
            assert np.all(d <= allow[name][0] * (1 + 1e-9)), (name, r, n, (d - allow[name][0]).max())
            moved = max(moved, d.max())
    assert moved > 0  # the planted flips did change the gradients


@pytest.mark.parametrize("call,name", [(4, "dw1"), (5, "dw3"), (6, "dw2"), (1, "dw2")])
def test_whole_term_errors_exceed_the_allowance(monkeypatch, call, name):
    case = _case(3)
    x, dy, w, dst_row, offsets, w1, w3, w2 = case
    allow = weight_grad_flip_allowance(dy, x, w, dst_row, offsets, w1, w3, w2)[name][0]
    base = _grads(case)[name]

    def drop_row(a):
        a[7] = 0.0
        return a

    def swap_rows(a):
        a[[3, 11]] = a[[11, 3]]
        return a

    def wrong_sign(a):  # on the row's largest term
        j = int(np.argmax(np.abs(a[5])))
        a[5, j] = -a[5, j]
        return a
    for edit in (drop_row, swap_rows, wrong_sign):
        got = _grads(case, monkeypatch, call, edit)[name]
        assert (np.abs(got - base) - allow).max() > 0, (call, name, edit.__name__)
