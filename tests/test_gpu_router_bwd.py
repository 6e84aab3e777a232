"""GPU parity of the router backward and the load-balance loss against the CPU
oracle.

Unit test (`test_router_bwd_unit`): moe_router_bwd alone on seeded inputs
that the oracle receives exactly (Yp, dY and dx_in are synthetic bf16/fp32
tensors, routing comes from the oracle): dL, dW_g, d(bias) and dX within
1e-4 * rms(ref) (fp32 sums over h and over tokens against fp64, the
cancellation in dL amplifying their rounding; dX plus its bf16 rounding).

Layer test (`test_router_backward`): forward, aux loss and backward of the
whole layer, routing fed the oracle's fp32 logits.  The router gradient goes
through dw = <dY, Yp> with the GPU's Yp computed from the bf16 A its forward
stored; an element of A whose exact value lies within fp32 rounding of a bf16
tie may round either way, and dL = w (dw - sum w dw) cancels, so per-element
dL is checked by the unit test, and the layer test checks the token sums dW_g
and d(bias) and the total dX, each twice:
  * max-norm, 2e-2 * rms(ref), against the oracle fed the same storage (A
    rounded to bf16 in its forward, `bf16_storage`);
  * rms, 1e-2 * rms(ref), against the exact fp64 oracle.
The aux loss must match within 1e-5 relative (an fp32 sum of T*E
probabilities).
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref

from test_gpu_parity import DEV, HALF_ULP_BF16, check_close, check_rms, dev_tensor, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16

CASES = [
    ("small", dict(T=300, h=256, h_ffn=384, E=8, k=2), 0.01, 1),
    ("e64_k6", dict(T=600, h=256, h_ffn=256, E=64, k=6), 0.02, 2),
    ("k1", dict(T=257, h=128, h_ffn=128, E=16, k=1), 0.05, 3),
    ("zipf", dict(T=700, h=256, h_ffn=256, E=32, k=3, zipf_s=1.2), 0.01, 4),
    ("e100_multi_chunk", dict(T=1100, h=384, h_ffn=128, E=100, k=4), 0.03, 5),
]


def _run(wl, inp, logits, alpha):
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_BF16,
                          backward=True)
    layer = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_BF16, save_for_backward=True)
    xd, wg = dev_tensor(inp["x"]), dev_tensor(inp["w_gate"])
    layer.forward(xd, wg, torch.from_numpy(inp["bias"]).to(DEV), P, logits_in=torch.from_numpy(logits).to(DEV))
    aux = layer.aux_loss(alpha)
    layer.backward(dev_tensor(inp["dy"]), xd, P, w_gate=wg, alpha=alpha)
    torch.cuda.synchronize()
    return layer, float(aux.cpu())


def _oracle(wl, inp, alpha):
    f = lambda k: to_f32(inp[k])
    x, wg = f("x"), f("w_gate")
    fw = ref.layer_forward(x, wg, inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    yp_st = ref.expert_forward(fw["xp"], fw["offsets"], f("w1"), f("w3"), f("w2"), keep=False,
                               bf16_storage=True)
    rb = ref.router_backward(f("dy"), fw["yp"][fw["dst_row"]], x, wg, fw["logits"], fw["idx"], fw["w"], alpha)
    rb_st = ref.router_backward(f("dy"), yp_st[fw["dst_row"]], x, wg, fw["logits"], fw["idx"], fw["w"], alpha)
    return fw, rb, rb_st


def _check2(got, ex, st, what):
    check_close(got, st, 2e-2, None, None, what + " vs bf16-storage oracle")
    check_rms(got, ex, 1e-2, what + " vs exact oracle")


@pytest.mark.parametrize("case,over,alpha,seed", CASES, ids=[c[0] for c in CASES])
def test_router_backward(case, over, alpha, seed):
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=case, **over)
    say(f"router backward {case}: {wl} alpha={alpha}")
    inp = moe_synth.gen_all(wl, seed=seed)
    fw, rb, rb_st = _oracle(wl, inp, alpha)
    layer, aux = _run(wl, inp, fw["logits"], alpha)
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), fw["dst_row"])
    want_aux = ref.aux_balance_loss(fw["logits"], fw["idx"], wl.E, wl.k, alpha)
    say(f"  aux loss gpu {aux:.8g} oracle {want_aux:.8g}")
    assert aux == pytest.approx(want_aux, rel=1e-5)
    _check2(layer.dw_gate.cpu().numpy(), rb["dw_gate"], rb_st["dw_gate"], "dW_g")
    _check2(layer.dbias.cpu().numpy(), rb["dbias"], rb_st["dbias"], "d(bias)")
    # the logit gradient of every token sums to zero (softmax shift invariance)
    dl = layer.dlogits.cpu().numpy().astype(np.float64)
    assert np.abs(dl.sum(axis=1)).max() <= 1e-4 * np.abs(dl).max()
    # total dX = expert path + router path
    f = lambda k: to_f32(inp[k])
    args = (f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], f("w1"), f("w3"), f("w2"))
    ex = ref.layer_backward(*args)["dx"] + rb["dx"]
    emu = ref.layer_backward(*args, bf16_operands=True)["dx"] + rb_st["dx"]
    out_round = HALF_ULP_BF16 * np.abs(emu)
    got = host(layer.dx)
    check_close(got, emu, 2e-2, None, None, "dX vs bf16-operand oracle", rounding=out_round)
    check_rms(got, ex, 1e-2, "dX vs exact oracle")


def test_top1_without_aux_has_zero_router_gradient():
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="k1a0", T=200, h=128, h_ffn=128, E=8, k=1)
    inp = moe_synth.gen_all(wl, seed=7)
    L = ref.router_logits(to_f32(inp["x"]), to_f32(inp["w_gate"]), inp["bias"])
    layer, aux = _run(wl, inp, L, 0.0)
    assert aux == 0.0
    assert not layer.dlogits.any() and not layer.dw_gate.any() and not layer.dbias.any()


def test_router_backward_deterministic():
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="det", T=900, h=256, h_ffn=128, E=16, k=2)
    inp = moe_synth.gen_all(wl, seed=8)
    L = ref.router_logits(to_f32(inp["x"]), to_f32(inp["w_gate"]), inp["bias"])
    a, aux_a = _run(wl, inp, L, 0.02)
    d1, g1, x1 = a.dlogits.clone(), a.dw_gate.clone(), a.dx.clone()
    b, aux_b = _run(wl, inp, L, 0.02)
    assert aux_a == aux_b
    assert torch.equal(d1, b.dlogits) and torch.equal(g1, b.dw_gate)
    assert torch.equal(x1.view(torch.int16), b.dx.view(torch.int16))


UNIT_CASES = [
    ("bf16_e8_k2", dict(T=333, h=256, E=8, k=2), 0.01, "bf16", 11),
    ("bf16_e64_k6", dict(T=600, h=128, E=64, k=6), 0.02, "bf16", 12),
    ("bf16_e100_k4", dict(T=700, h=192, E=100, k=4), 0.03, "bf16", 13),
    ("bf16_k1", dict(T=129, h=64, E=16, k=1), 0.05, "bf16", 14),
    ("f32_e8_k2", dict(T=257, h=128, E=8, k=2), 0.01, "f32", 15),
    # one expert: dL, dW_g and d(bias) are exactly zero
    ("bf16_e1", dict(T=163, h=256, E=1, k=1), 0.03, "bf16", 16),
]


@pytest.mark.parametrize("case,sh,alpha,st,seed", UNIT_CASES, ids=[c[0] for c in UNIT_CASES])
def test_router_bwd_unit(case, sh, alpha, st, seed):
    T, h, E, k = sh["T"], sh["h"], sh["E"], sh["k"]
    say(f"router bwd unit {case}: T={T} h={h} E={E} k={k} alpha={alpha} {st}")
    g = lambda name, shape, std=1.0, stor=st: moe_synth.gen_matrix(name, shape, std, stor, seed)
    x, dy = g("x", (T, h)), g("dy", (T, h))
    wg = g("w_gate", (h, E), 0.05)
    yp = g("yp", (T * k, h))
    dx_in = g("dx_in", (T, h), 1.0, "f32")
    f = lambda a: to_f32(a).astype(np.float64)
    L = ref.router_logits(f(x), f(wg), None)
    idx, w = ref.topk_softmax(L, k)
    counts, offsets, dst_row, src_tok = ref.build_index(idx, E)
    rb = ref.router_backward(f(dy), f(yp)[dst_row], f(x), f(wg), L, idx, w, alpha)
    # the GPU's own routing from the same logits (bit-exact ids, w to 1e-6)
    tdt = torch.float32 if st == "f32" else torch.bfloat16
    dev = lambda a: dev_tensor(a)
    d_idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    d_w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    d_L = torch.from_numpy(L.astype(np.float32)).to(DEV)
    code = ops.dtype_code(tdt)
    ops.moe_route(None, None, None, d_L, T, h, E, k, code, d_idx, d_w)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    out = dict(dx=torch.empty(T, h, dtype=tdt, device=DEV),
               dL=torch.empty(T, E, dtype=torch.float32, device=DEV),
               dwg=torch.empty(h, E, dtype=torch.float32, device=DEV),
               db=torch.empty(E, dtype=torch.float32, device=DEV))
    wsb = ops.moe_router_bwd_workspace_size(T, h, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    ops.moe_router_bwd(dev(dy), dev(yp), code, i32(dst_row), d_idx, d_w, d_L, i32(counts), T, h, E, k, alpha,
                       code, dev(x), dev(wg), torch.from_numpy(dx_in).to(DEV), out["dx"], out["dL"],
                       out["dwg"], out["db"], ws, wsb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_idx.cpu().numpy(), idx)
    check_close(out["dL"].cpu().numpy(), rb["dL"], 1e-4, None, None, "dL")
    check_close(out["dwg"].cpu().numpy(), rb["dw_gate"], 1e-4, None, None, "dW_g")
    check_close(out["db"].cpu().numpy(), rb["dbias"], 1e-4, None, None, "d(bias)")
    want_dx = dx_in.astype(np.float64) + rb["dx"]
    rnd = HALF_ULP_BF16 * np.abs(want_dx) if st == "bf16" else None
    check_close(host(out["dx"]), want_dx, 1e-4, None, None, "dX", rounding=rnd)
