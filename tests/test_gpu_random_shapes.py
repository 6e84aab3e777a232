"""GPU parity on seeded random shapes: the layer forward and backward (BF16),
the FP8 forward, the FP8 backward, the router backward and the tile-arrival
forward (against the plain entries, bit for bit, on the GPU's own routing); the
others with routing fed the oracle's fp32 logits.

Shapes are drawn per seed: T from 1 to 700, h and h_ffn in {128, 256, 384}
(one to three 128-wide blocks, so tiles end ragged in every dimension), E from
1 to 47, k from 1 to min(E, 8), with or without a Zipf router bias (experts
without rows appear).  The bars are those of the fixed-shape tests: routing,
index and dispatch bit-exact; y within 2e-2 * rms of the oracle (plus y's
own bf16 rounding); the gradients within 2e-2 * rms (max-norm) of the oracle
with BF16 operands and within 1e-2 * rms (rms) of the exact oracle; against
the BF16-operand oracle the weight gradients also allow, per element, the
largest change one operand rounded to the neighbouring BF16 value makes
(`bf16_flip`: an fp32 and an fp64 value on either side of a BF16 rounding
boundary; seeds 48, 91, 132 and 134 are shapes where that happened), and at
most a small fraction of elements may need it; the FP8 forward at 6e-2 * rms with the oracle's allowance
for fp32 implementations (`check_fp8_forward`), the FP8 backward likewise
against its allowance; the router backward within 1e-4 * rms; experts without
rows get zero weight gradients.
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref

from test_gpu_parity import (HALF_ULP_BF16, _run_gpu_layer, check_close, check_fp8_forward, check_rms, host,
                             say, y_rounding)
from test_gpu_backward import _gpu_fwd_bwd
from bf16_flip import weight_grad_flip_allowance

pytestmark = pytest.mark.gpu


def _shape(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 48))
    return dict(T=int(rng.integers(1, 701)), h=int(rng.choice([128, 256, 384])),
                h_ffn=int(rng.choice([128, 256, 384])), E=E, k=int(rng.integers(1, min(E, 8) + 1)),
                zipf_s=float(rng.choice([0.0, 1.2])))


@pytest.mark.parametrize("seed", list(range(12)) + [48, 91, 132, 134])
def test_random_shape_forward_backward(seed):
    over = _shape(seed)
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=f"rand{seed}", **over)
    say(f"random shape {seed}: {wl}")
    inp = moe_synth.gen_all(wl, seed=seed)
    f = lambda k: to_f32(inp[k])
    fw = ref.layer_forward(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    layer = _gpu_fwd_bwd(wl, inp, fw["logits"])
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), fw["idx"])
    np.testing.assert_array_equal(layer.counts.cpu().numpy(), fw["counts"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), fw["offsets"])
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), fw["dst_row"])
    check_close(host(layer.y), fw["y"], 2e-2, None, None, "y", rounding=y_rounding(fw["y"]))
    args = (f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], f("w1"), f("w3"), f("w2"))
    bw = ref.layer_backward(*args)
    emu = ref.layer_backward(*args, bf16_operands=True)
    flip = weight_grad_flip_allowance(*args)
    got = {"dx": host(layer.dx), "dw1": layer.dw1.cpu().numpy(), "dw3": layer.dw3.cpu().numpy(),
           "dw2": layer.dw2.cpu().numpy()}
    for name in ("dx", "dw1", "dw3", "dw2"):
        if not np.any(emu[name]):
            assert not np.any(got[name]), name
            continue
        if name == "dx":
            check_close(got[name], emu[name], 2e-2, None, None, name + " vs bf16-operand oracle",
                        rounding=HALF_ULP_BF16 * np.abs(emu[name]))
        else:
            check_close(got[name], emu[name], 2e-2, flip[name], None, name + " vs bf16-operand oracle")
        check_rms(got[name], bw[name], 1e-2, name + " vs exact oracle")
    for e in np.nonzero(fw["counts"] == 0)[0]:
        assert not layer.dw1[e].any() and not layer.dw3[e].any() and not layer.dw2[e].any()


@pytest.mark.parametrize("seed", range(4))
def test_random_shape_forward_fp8(seed):
    over = _shape(20 + seed)
    wl = moe_synth.WORKLOADS["tiny"].scaled(name=f"rand_fp8_{seed}", dtype="fp8", **over)
    say(f"random shape fp8 {seed}: {wl}")
    inp = moe_synth.gen_all(wl, seed=seed)
    f = lambda k: to_f32(inp[k])
    r = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    layer, _ = _run_gpu_layer(wl, inp, logits_in=r["logits"])
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), r["idx"])
    np.testing.assert_array_equal(layer.xp.cpu().numpy()[: wl.T * wl.k], ref.permute(r["qx"], r["dst_row"]))
    check_fp8_forward(layer, wl, r, f)


@pytest.mark.parametrize("seed", range(4))
def test_random_shape_fp8_backward(seed):
    """FP8 backward on shared G|U and gate weights (the unit form of the FP8
    backward test, with the oracle's allowance)."""
    from test_gpu_backward_fp8 import _check, _run
    over = _shape(40 + seed)
    over.pop("zipf_s")
    _check(*_run(f"rand_bwd_fp8_{seed}", over, seed, True))


@pytest.mark.parametrize("seed", range(4))
def test_random_shape_router_backward(seed):
    """Router backward on inputs the oracle receives exactly (the unit form
    of the router backward test), BF16 storage, balance-loss weight 0.03."""
    from test_gpu_router_bwd import test_router_bwd_unit
    sh = _shape(60 + seed)
    test_router_bwd_unit(f"rand_router_{seed}", dict(T=sh["T"], h=sh["h"], E=sh["E"], k=sh["k"]), 0.03,
                         "bf16", 70 + seed)


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_fp8_token_gather_bit_identical(seed):
    """The FP8 backward's two entry points (operands gathered from dY and x,
    or read from their dispatched bf16 copies) agree bit for bit."""
    from test_gpu_backward_fp8 import gather_entry_matches
    over = _shape(100 + seed)
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=f"randg{seed}", dtype="fp8", **over)
    say(f"random shape (FP8 gather) {seed}: {wl}")
    gather_entry_matches(wl, moe_synth.gen_all(wl, seed=seed))


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_arrival_bit_identical(seed):
    """The tile-arrival forward (copy beside FC1, per-expert flags) equals
    moe_permute + moe_grouped_swiglu_fwd bit for bit, with no wait giving up."""
    from test_gpu_arrival import _compare
    over = _shape(200 + seed)
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=f"randa{seed}", **over)
    say(f"random shape (tile arrival) {seed}: {wl}")
    _compare(wl, moe_synth.gen_all(wl, seed=seed))
