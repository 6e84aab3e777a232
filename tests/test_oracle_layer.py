"""Pins for the oracle's expert FFN and whole forward layer.

Pins: a hand-computed scalar case (closed form with math.exp), the E = 1,
k = 1 reduction to a dense SwiGLU FFN evaluated with torch's CPU ``silu``,
the per-token (un-permuted) form, and zero / linearity special cases.
"""
import math

import numpy as np
import pytest
import torch

import moe_synth
from oracle import moe_ref as ref


def test_scalar_closed_form():
    # T=1, h=1, h_ffn=1, E=2, k=1: y = SiLU(x*w1) * (x*w3) * w2 of the chosen expert
    x = np.array([[1.5]], np.float32)
    wg = np.array([[1.0, -1.0]], np.float32)      # expert 0 wins for x > 0
    w1 = np.array([[[0.5]], [[9.0]]]); w3 = np.array([[[-2.0]], [[9.0]]]); w2 = np.array([[[0.25]], [[9.0]]])
    out = ref.layer_forward(x, wg, None, w1, w3, w2, k=1)
    g = 0.75
    want = g / (1 + math.exp(-g)) * (1.5 * -2.0) * 0.25
    assert out["idx"].tolist() == [[0]] and out["w"].tolist() == [[1.0]]
    assert out["y"][0, 0] == pytest.approx(want, rel=1e-15)
    # negative input routes to expert 1
    out = ref.layer_forward(-x, wg, None, w1, w3, w2, k=1)
    g = -1.5 * 9.0
    assert out["idx"].tolist() == [[1]]
    assert out["y"][0, 0] == pytest.approx(g / (1 + math.exp(-g)) * (-1.5 * 9.0) * 9.0, rel=1e-14)


def test_single_expert_is_dense_swiglu():
    rng = np.random.default_rng(0)
    T, h, hf = 17, 24, 40
    x = rng.standard_normal((T, h)); wg = rng.standard_normal((h, 1))
    w1 = rng.standard_normal((1, h, hf)) / 5; w3 = rng.standard_normal((1, h, hf)) / 5
    w2 = rng.standard_normal((1, hf, h)) / 6
    out = ref.layer_forward(x, wg, None, w1, w3, w2, k=1)
    xt = torch.from_numpy(x)
    dense = (torch.nn.functional.silu(xt @ torch.from_numpy(w1[0])) * (xt @ torch.from_numpy(w3[0]))) @ torch.from_numpy(w2[0])
    np.testing.assert_allclose(out["y"], dense.numpy(), rtol=1e-12, atol=1e-12)


def test_permuted_matches_per_token_form():
    wl = moe_synth.WORKLOADS["tiny"]
    inp = moe_synth.gen_all(wl, seed=0)
    out = ref.layer_forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], wl.k)
    yt = ref.layer_forward_tokens(inp["x"], out["idx"], out["w"], inp["w1"], inp["w3"], inp["w2"])
    np.testing.assert_allclose(out["y"], yt, rtol=1e-12, atol=1e-12 * np.abs(yt).max())
    assert out["counts"].sum() == wl.T * wl.k
    assert out["y"].shape == (wl.T, wl.h)


def test_zero_gate_or_up_gives_zero():
    rng = np.random.default_rng(1)
    T, h, hf, E = 9, 8, 12, 3
    x = rng.standard_normal((T, h)); wg = rng.standard_normal((h, E))
    w = rng.standard_normal((E, h, hf)); w2 = rng.standard_normal((E, hf, h))
    assert np.all(ref.layer_forward(x, wg, None, np.zeros_like(w), w, w2, 2)["y"] == 0)
    assert np.all(ref.layer_forward(x, wg, None, w, np.zeros_like(w), w2, 2)["y"] == 0)


def test_linear_in_down_projection_and_up():
    rng = np.random.default_rng(2)
    T, h, hf, E = 11, 8, 12, 4
    x = rng.standard_normal((T, h)); wg = rng.standard_normal((h, E))
    w1 = rng.standard_normal((E, h, hf)); w3 = rng.standard_normal((E, h, hf)); w2 = rng.standard_normal((E, hf, h))
    y = ref.layer_forward(x, wg, None, w1, w3, w2, 2)["y"]
    np.testing.assert_allclose(ref.layer_forward(x, wg, None, w1, w3, 3 * w2, 2)["y"], 3 * y, rtol=1e-13)
    np.testing.assert_allclose(ref.layer_forward(x, wg, None, w1, -w3, w2, 2)["y"], -y, rtol=1e-13)


def test_bias_shifts_routing():
    wl = moe_synth.WORKLOADS["m352b_zipf"]
    _, bias = moe_synth.gen_router(wl.scaled(h=8), seed=0)
    p = np.exp(bias.astype(np.float64))
    np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-6)
    assert np.all(np.diff(bias) < 0)
    # with zero gate weights the bias alone decides: everyone picks experts 0..k-1
    L = ref.router_logits(np.ones((4, 8), np.float32), np.zeros((8, wl.E), np.float32), bias)
    idx, _ = ref.topk_softmax(L, wl.k)
    assert idx.tolist() == [[0, 1, 2]] * 4
