"""Pins for the oracle's backward: central finite differences in fp64 and
torch CPU autograd of the per-token form (routing held fixed)."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as ref


def _setup(seed=0, T=6, h=5, hf=4, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h)); wg = rng.standard_normal((h, E))
    w1 = rng.standard_normal((E, h, hf)) * 0.7; w3 = rng.standard_normal((E, h, hf)) * 0.7
    w2 = rng.standard_normal((E, hf, h)) * 0.7; dy = rng.standard_normal((T, h))
    fw = ref.layer_forward(x, wg, None, w1, w3, w2, k)
    return x, w1, w3, w2, dy, fw


def _loss(x, w1, w3, w2, dy, fw):
    xp = ref.permute(x, fw["dst_row"])
    yp = ref.expert_forward(xp, fw["offsets"], w1, w3, w2, keep=False)
    return float(np.sum(ref.combine(yp, fw["dst_row"], fw["w"]) * dy))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    x, w1, w3, w2, dy, fw = _setup(seed)
    bw = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2)
    eps = 1e-6
    for name, arr, grad in (("x", x, bw["dx"]), ("w1", w1, bw["dw1"]), ("w3", w3, bw["dw3"]), ("w2", w2, bw["dw2"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x, "w1": w1, "w3": w3, "w2": w2}
            plus = {k2: v.copy() for k2, v in args.items()}
            minus = {k2: v.copy() for k2, v in args.items()}
            plus[name][i] += eps; minus[name][i] -= eps
            num[i] = (_loss(plus["x"], plus["w1"], plus["w3"], plus["w2"], dy, fw)
                      - _loss(minus["x"], minus["w1"], minus["w3"], minus["w2"], dy, fw)) / (2 * eps)
        scale = np.abs(num).max()
        assert scale > 0
        assert np.abs(num - grad).max() <= 1e-6 * scale, name


def test_per_token_and_per_expert_forms_match():
    x, w1, w3, w2, dy, fw = _setup(7, T=11, h=6, hf=5, E=4, k=2)
    bw = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2)
    dx = ref.layer_backward_tokens(dy, x, fw["idx"], fw["w"], w1, w3, w2)
    np.testing.assert_allclose(dx, bw["dx"], rtol=1e-12, atol=1e-13)
    xp = ref.permute(x, fw["dst_row"])
    dyp = ref.permute(dy, fw["dst_row"], row_scale=fw["w"])
    for e in range(4):
        lo, hi = fw["offsets"][e], fw["offsets"][e + 1]
        g1, g3, g2, dxp = ref.expert_grads(xp[lo:hi], dyp[lo:hi], w1[e], w3[e], w2[e])
        np.testing.assert_allclose(g1, bw["dw1"][e], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g3, bw["dw3"][e], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2, bw["dw2"][e], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dxp, bw["dxp"][lo:hi], rtol=1e-12, atol=1e-13)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.uniform(-5, 5, 10000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)]])
    want = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref.round_bf16(v), want)


def test_bf16_operand_emulation_consistent():
    x, w1, w3, w2, dy, fw = _setup(4, T=13, h=6, hf=5, E=3, k=2)
    exact = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2)
    emu = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, bf16_operands=True)
    dx = ref.layer_backward_tokens(dy, x, fw["idx"], fw["w"], w1, w3, w2, bf16_operands=True)
    np.testing.assert_allclose(dx, emu["dx"], rtol=1e-12, atol=1e-13)
    for k in ("dx", "dw1", "dw3", "dw2"):
        rel = np.abs(emu[k] - exact[k]).max() / np.abs(exact[k]).max()
        assert 0 < rel < 2e-2, k            # rounding happened, and is small


def test_backward_matches_torch_autograd():
    x, w1, w3, w2, dy, fw = _setup(5, T=9, h=6, hf=7, E=4, k=3)
    bw = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2)
    tx = torch.tensor(x, requires_grad=True)
    t1 = torch.tensor(w1, requires_grad=True); t3 = torch.tensor(w3, requires_grad=True)
    t2 = torch.tensor(w2, requires_grad=True)
    idx = torch.tensor(fw["idx"].astype(np.int64)); wt = torch.tensor(fw["w"].astype(np.float64))
    y = torch.zeros_like(tx)
    for j in range(idx.shape[1]):
        e = idx[:, j]
        g = torch.einsum("th,thf->tf", tx, t1[e]); u = torch.einsum("th,thf->tf", tx, t3[e])
        y = y + wt[:, j:j + 1] * torch.einsum("tf,tfh->th", torch.nn.functional.silu(g) * u, t2[e])
    (y * torch.tensor(dy)).sum().backward()
    for got, want in ((bw["dx"], tx.grad), (bw["dw1"], t1.grad), (bw["dw3"], t3.grad), (bw["dw2"], t2.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)
    # saved-activation path gives the same result as recomputing from x
    bw2 = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, g=fw["g"], u=fw["u"])
    np.testing.assert_allclose(bw2["dw1"], bw["dw1"], rtol=1e-13)
