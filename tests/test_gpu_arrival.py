"""Dispatch copy and FC1 overlapped by tile arrival (moe_dispatch_swiglu_fwd):
the same index, routed rows, kept G|U, expert outputs and layer output as
moe_permute followed by moe_grouped_swiglu_fwd, bit for bit, and a status of
0 (no wait of FC1 for its rows gave up).  The GEMM arithmetic is the same in
both, so any difference would be a row that FC1 read before the copy had
released it, or a block count that never completed."""
import numpy as np
import pytest
import torch

import moe_synth

from test_gpu_parity import DEV, dev_tensor, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16

CASES = [
    ("small", dict(T=300, h=256, h_ffn=384, E=8, k=2), 1),
    ("e64_k6", dict(T=600, h=256, h_ffn=256, E=64, k=6), 2),
    # many rounds of row tiles, so FC1's waits span the copy
    ("multi_round", dict(T=4096, h=512, h_ffn=1024, E=8, k=2), 3),
    ("zipf_empty", dict(T=300, h=256, h_ffn=256, E=16, k=2, zipf_s=2.5), 4),
    ("one_token", dict(T=1, h=256, h_ffn=128, E=4, k=2), 5),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _compare(wl, inp, repeats=2, **fwd):
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_BF16)
    x, wg = dev_tensor(inp["x"]), dev_tensor(inp["w_gate"])
    bias = torch.from_numpy(inp["bias"]).to(DEV)
    ref = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_BF16, save_for_backward=True)
    arr = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_BF16, save_for_backward=True)
    ref.forward(x, wg, bias, P, **fwd)
    for rep in range(repeats):  # the flags are cleared by each call
        arr.forward(x, wg, bias, P, arrival=True, **fwd)
        torch.cuda.synchronize()
        assert int(arr.arrival_status.item()) == 0, "a wait of FC1 for its rows gave up"
        kept = int(ref.offsets[wl.E])
        for n in ("topk_idx", "counts", "offsets", "dst_row", "y"):
            assert torch.equal(_bits(getattr(arr, n)), _bits(getattr(ref, n))), (n, rep)
        for n in ("src_tok", "xp", "h13", "yp"):
            assert torch.equal(_bits(getattr(arr, n)[:kept]), _bits(getattr(ref, n)[:kept])), (n, rep)


@pytest.mark.parametrize("case,over,seed", CASES, ids=[c[0] for c in CASES])
def test_arrival_forward_bit_identical(case, over, seed):
    wl = moe_synth.WORKLOADS["mixtral"].scaled(name=case, **over)
    say(f"tile arrival {case}: {wl}")
    _compare(wl, moe_synth.gen_all(wl, seed=seed))


def test_arrival_forward_with_capacity_drop():
    """Pairs dropped by capacity (ids set to -1) are left out of the copy's
    row counts as of the index: FC1 must still see every expert complete."""
    wl = moe_synth.WORKLOADS["mixtral"].scaled(name="capacity", T=1024, h=256, h_ffn=256, E=8, k=2)
    say(f"tile arrival with capacity 160 (mean 256 pairs per expert): {wl}")
    _compare(wl, moe_synth.gen_all(wl, seed=6), capacity=160)


def test_arrival_wait_gives_up_without_copy():
    """FC1's waits are bounded: with the copy left out and a 64-poll limit
    (the wait self-test entry) every wait gives up, the kernels end and the
    status reads 1; the next real call clears it and matches the plain path."""
    wl = moe_synth.WORKLOADS["mixtral"].scaled(name="wait", T=300, h=256, h_ffn=384, E=8, k=2)
    say(f"tile arrival, waits forced to give up: {wl}")
    inp = moe_synth.gen_all(wl, seed=7)
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_BF16)
    x, wg = dev_tensor(inp["x"]), dev_tensor(inp["w_gate"])
    bias = torch.from_numpy(inp["bias"]).to(DEV)
    ref = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_BF16, save_for_backward=True)
    arr = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_BF16, save_for_backward=True)
    ref.forward(x, wg, bias, P)
    arr.forward(x, wg, bias, P, arrival=True)
    torch.cuda.synchronize()
    assert int(arr.arrival_status.item()) == 0
    ops.moe_dispatch_swiglu_fwd_wait_selftest(x, arr.topk_idx, wl.T, wl.k, arr.counts, arr.offsets, arr.dst_row,
                                              arr.src_tok, P.struct, arr.xp, arr.h13, arr.yp, arr.yp_code,
                                              arr.arrival_status, arr.aws, arr.aws_bytes)
    torch.cuda.synchronize()
    assert int(arr.arrival_status.item()) == 1, "a wait with no copy beside it did not give up"
    arr.forward(x, wg, bias, P, arrival=True)
    torch.cuda.synchronize()
    assert int(arr.arrival_status.item()) == 0
    assert torch.equal(_bits(arr.y), _bits(ref.y))


@pytest.mark.slow
def test_arrival_forward_full_size_mixtral():
    """The Mixtral-shaped layer (T 8192, h 4096, h_ffn 14336, E 8, k 2)."""
    wl = moe_synth.WORKLOADS["mixtral"]
    say("tile arrival, full-size Mixtral shape")
    _compare(wl, moe_synth.gen_all(wl, seed=0), repeats=1)
