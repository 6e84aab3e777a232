"""GPU parity of the FP8 backward against the quantization-emulating oracle.

Forward in FP8 (kept G|U in bf16), backward on E4M3 codes (see the oracle's
`layer_backward_fp8` for the recipe); routing fed the oracle's fp32 logits.

A quantizer turns the last-bit differences of fp32 vs fp64 arithmetic before
it into whole code steps (up to 1/8 of a value, or a new scale for a whole
row when the row's amax moves), so two correct implementations differ by more
than the FP8 bar on a few elements.  The oracle's `fp8_backward_envelope`
bounds, per element, the distance of any implementation with fp32 sums and
an fp32 SwiGLU derivative from `layer_backward_fp8`; each of dX, dW1, dW3,
dW2 must be within 6e-2 * rms of the emulating oracle once that allowance is
granted (dX also half a bf16 ulp of its own output rounding), and its rms
error below 1e-2 * rms.

Unit test (`test_fp8_backward_unit`): the GPU backward gets the oracle's
G|U (rounded to bf16, in the packed column order) in place of the kept
forward output and the oracle's fp32 gate weights in place of its own; the
envelope is tight (mean allowance ~1e-3 * rms for dW).
Layer test (`test_fp8_backward_layer`): the GPU's own forward and router
feed the backward; the envelope includes the forward's fp32 error on G, U
and the fp32 softmax's on the gate weights.

The FP8 backward weight copies are compared code for code with the oracle's
per-row quantization.  Experts without rows get zero weight gradients, also
when no expert has rows (rows = 0, FP8 and BF16).
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref

import fp8_sub
from test_gpu_parity import DEV, HALF_ULP_BF16, check_close, dev_tensor, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16, MOE_FP8_E4M3

CASES = [
    ("small", dict(T=300, h=256, h_ffn=384, E=8, k=2), 1),
    ("tail_n", dict(T=513, h=384, h_ffn=256, E=4, k=2), 2),
    ("e64_k6", dict(T=600, h=256, h_ffn=256, E=64, k=6), 3),
    ("multi_tile", dict(T=2100, h=512, h_ffn=384, E=4, k=2), 4),
    ("one_expert", dict(T=77, h=256, h_ffn=128, E=1, k=1), 6),
    ("zipf_empty", dict(T=300, h=256, h_ffn=256, E=16, k=2, zipf_s=2.5), 7),
    # dG|dU has 2816 columns: 44 strips x 64 experts = 2816 transpose work
    # items, more than the transposes' bounded grid, so workgroups take several
    ("many_strips", dict(T=200, h=256, h_ffn=1408, E=64, k=6), 8),
]


def test_fp8_backward_weight_copies():
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="packq", T=16, h=256, h_ffn=384, E=3, k=2)
    inp = moe_synth.gen_all(wl, seed=3)
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_FP8_E4M3,
                          backward=True)
    torch.cuda.synchronize()
    E, h, hf = wl.E, wl.h, wl.h_ffn
    w2b = P.w2_bwd.cpu().numpy().reshape(E, hf, h)
    w13b = P.w13_bwd.cpu().numpy().reshape(E, h, 2 * hf)
    for e in range(E):
        q, s = ref.quantize_weight_rows(to_f32(inp["w2"][e]))                 # rows = h_ffn channels
        np.testing.assert_array_equal(w2b[e], q)
        np.testing.assert_array_equal(P.w2_bwd_scale[e].cpu().numpy(), s)
        cat = np.concatenate([to_f32(inp["w1"][e]), to_f32(inp["w3"][e])], axis=1)   # [h, 2hf]
        q, s = ref.quantize_weight_rows(cat)
        np.testing.assert_array_equal(P.w13_bwd_scale[e].cpu().numpy(), s)
        p = np.arange(2 * hf)
        src = np.where((p // 32) % 2 == 1, hf, 0) + (p // 64) * 32 + p % 32   # interleaved column p
        np.testing.assert_array_equal(w13b[e], q[:, src])


def _packed_gu(g, u):
    """[rows][2hf] G|U with 32-column groups of G and U interleaved (the
    packed order of the kept forward output)."""
    return np.concatenate([g, u], axis=1)[:, fp8_sub.gu_src_columns(g.shape[1])]


def _check(got, emu, exact, allow):
    for name in ("dx", "dw1", "dw3", "dw2"):
        extra = HALF_ULP_BF16 * np.abs(emu[name]) if name == "dx" else 0.0
        rms = np.sqrt(np.mean(emu[name] ** 2))
        say(f"  {name}: allowance / rms mean {np.mean(allow[name]) / rms:.2e} max {np.max(allow[name]) / rms:.2e}")
        check_close(got[name], emu[name], 6e-2, allow[name], None, name + " vs FP8-emulating oracle",
                    rounding=extra)
        e_rms = np.sqrt(np.mean((got[name] - emu[name]) ** 2)) / rms
        x_rms = np.sqrt(np.mean((got[name] - exact[name]) ** 2)) / np.sqrt(np.mean(exact[name] ** 2))
        say(f"  {name}: rms err / rms vs emulating oracle {e_rms:.3e}, vs exact {x_rms:.3e}")
        assert e_rms <= 1e-2, name


def _run(case, over, seed, shared_gu):
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=case, dtype="fp8", **over)
    say(f"fp8 backward {case}: {wl} shared G|U={shared_gu}")
    inp = moe_synth.gen_all(wl, seed=seed)
    f = lambda key: to_f32(inp[key])
    fw = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    args = (f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], f("w1"), f("w3"), f("w2"), fw["g"], fw["u"])
    emu = ref.layer_backward_fp8(*args)
    if shared_gu:
        g_err = u_err = w_err = None
    else:
        g_err, u_err = ref.fp8_forward_gu_bound(f("x"), fw["dst_row"], fw["offsets"], f("w1"), f("w3"))
        w_err = ref.topk_weight_bound(fw["logits"], fw["idx"])
    allow = ref.fp8_backward_envelope(*args, g_err=g_err, u_err=u_err, w_err=w_err)
    exact = ref.layer_backward(f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], f("w1"), f("w3"), f("w2"),
                               g=fw["g"], u=fw["u"])
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_FP8_E4M3,
                          backward=True)
    layer = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_FP8_E4M3, save_for_backward=True)
    xd = dev_tensor(inp["x"])
    layer.forward(xd, dev_tensor(inp["w_gate"]), torch.from_numpy(inp["bias"]).to(DEV), P,
                  logits_in=torch.from_numpy(fw["logits"]).to(DEV))
    if shared_gu:
        gu = _packed_gu(np.asarray(fw["g"], np.float64), np.asarray(fw["u"], np.float64))
        layer.h13.copy_(torch.from_numpy(gu.astype(np.float32)).to(DEV).to(torch.bfloat16))
        layer.topk_w.copy_(torch.from_numpy(np.asarray(fw["w"], np.float32)).to(DEV))
    layer.backward(dev_tensor(inp["dy"]), xd, P)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), fw["dst_row"])
    got = {"dx": host(layer.dx), "dw1": layer.dw1.cpu().numpy(), "dw3": layer.dw3.cpu().numpy(),
           "dw2": layer.dw2.cpu().numpy()}
    # experts without rows: zero weight gradients, exactly
    for e in np.nonzero(np.diff(fw["offsets"]) == 0)[0]:
        for name in ("dw1", "dw3", "dw2"):
            assert not got[name][e].any(), (name, e)
    return got, emu, exact, allow


@pytest.mark.parametrize("case,over,seed", CASES, ids=[c[0] for c in CASES])
def test_fp8_backward_unit(case, over, seed):
    _check(*_run(case, over, seed, True))


@pytest.mark.parametrize("case,over,seed", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_fp8_backward_layer(case, over, seed):
    _check(*_run(case, over, seed, False))


def test_fp8_backward_has_empty_experts_case():
    """The zipf_empty case does route no token to some experts."""
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="zipf_empty", dtype="fp8", T=300, h=256, h_ffn=256, E=16, k=2,
                                             zipf_s=2.5)
    inp = moe_synth.gen_all(wl, seed=7)
    L = ref.router_logits(to_f32(inp["x"]), to_f32(inp["w_gate"]), inp["bias"])
    idx, _ = ref.topk_softmax(L, wl.k)
    assert (np.bincount(idx.ravel(), minlength=wl.E) == 0).any()


@pytest.mark.parametrize("form", ["fp8", "fp8_tok", "bf16"])
def test_backward_no_rows(form):
    """rows = 0: no error, and every expert's weight gradient is written as
    zeros (fp8_tok: every pair of three tokens dropped)."""
    fp8 = form != "bf16"
    E, h, hf = 4, 256, 128
    rng = np.random.default_rng(0)
    w = lambda *sh: torch.from_numpy((rng.standard_normal(sh) * 0.05).astype(np.float32)).to(DEV).to(torch.bfloat16)
    code = MOE_FP8_E4M3 if fp8 else MOE_BF16
    P = ops.PackedWeights(w(E, h, hf), w(E, h, hf), w(E, hf, h), code, backward=True)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    dummy8 = torch.zeros(256, dtype=torch.uint8, device=DEV)
    dummyf = torch.zeros(64, dtype=torch.float32, device=DEV)
    dummyb = torch.zeros(128, dtype=torch.bfloat16, device=DEV)
    dw1 = torch.full((E, h, hf), float("nan"), device=DEV)
    dw3 = torch.full((E, h, hf), float("nan"), device=DEV)
    dw2 = torch.full((E, hf, h), float("nan"), device=DEV)
    if form == "fp8_tok":
        wsb = ops.moe_grouped_bwd_fp8_workspace_size(0, h, hf, E)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
        T, k = 3, 2
        tok = torch.zeros(T, h, dtype=torch.bfloat16, device=DEV)
        dst_row = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
        topk_w = torch.full((T, k), 0.5, dtype=torch.float32, device=DEV)
        ops.moe_grouped_swiglu_bwd_fp8_tok(dummy8, dummyf, tok, tok, dst_row, topk_w, T, k, dummyb, P.struct,
                                           offsets, 0, dummyb, dw1, dw3, dw2, ws, ws.numel())
    elif fp8:
        wsb = ops.moe_grouped_bwd_fp8_workspace_size(0, h, hf, E)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
        ops.moe_grouped_swiglu_bwd_fp8(dummy8, dummyf, dummyb, dummyb, dummyb, P.struct, offsets, 0, dummyb, dw1,
                                       dw3, dw2, ws, ws.numel())
    else:
        wsb = ops.moe_grouped_bwd_workspace_size(0, h, hf, E, MOE_BF16)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
        ops.moe_grouped_swiglu_bwd(dummyb, dummyb, dummyb, P.struct, offsets, 0, dummyb, dw1, dw3, dw2, ws,
                                   ws.numel())
    torch.cuda.synchronize()
    for t in (dw1, dw3, dw2):
        assert torch.equal(t, torch.zeros_like(t))



@pytest.mark.slow
def test_full_size_dsmoe_fp8_backward_sampled():
    """The DeepSeekMoE-shaped FP8 backward at full size (T 16384, h 2048,
    h_ffn 1408, E 64, k 6), in the launch configuration the benchmark times.
    The oracle runs on sub-problems whose FP8 quantizers see exactly the
    values they see in the whole layer (`fp8_sub`): every routed row of one
    expert, for three experts, gives their complete dW1, dW3, dW2; the routed
    rows of 32 sampled tokens give their dX.  Both take the GPU's kept G|U and
    gate weights (the unit test's setting, so the envelope needs no forward
    error terms) and the FP8 bars of the small cases."""
    wl = moe_synth.WORKLOADS["dsmoe_fp8"]
    say("full-size dsmoe fp8 backward: generating inputs")
    inp = moe_synth.gen_all(wl, seed=0)
    x32, dy32 = to_f32(inp["x"]), to_f32(inp["dy"])
    L = ref.router_logits(x32, to_f32(inp["w_gate"]), inp["bias"])
    idx, _ = ref.topk_softmax(L, wl.k)
    say("full-size dsmoe fp8 backward: gpu")
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_FP8_E4M3,
                          backward=True)
    layer = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, MOE_FP8_E4M3, save_for_backward=True)
    xd = dev_tensor(inp["x"])
    layer.forward(xd, dev_tensor(inp["w_gate"]), torch.from_numpy(inp["bias"]).to(DEV), P,
                  logits_in=torch.from_numpy(L).to(DEV))
    layer.backward(dev_tensor(inp["dy"]), xd, P)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), idx)
    offsets, dst_row, src_tok = (layer.offsets.cpu().numpy(), layer.dst_row.cpu().numpy(),
                                 layer.src_tok.cpu().numpy())
    w_gpu = layer.topk_w.cpu().numpy()
    g_rows, u_rows = fp8_sub.unpack_gu(host(layer.h13))
    W = [to_f32(inp[n]) for n in ("w1", "w3", "w2")]
    got_w = {n: getattr(layer, n).cpu().numpy() for n in ("dw1", "dw3", "dw2")}

    def oracle(toks, slots, experts):
        args = fp8_sub.subproblem(dy32, x32, w_gpu, idx, dst_row, g_rows, u_rows, *W, toks, slots, experts)
        return (ref.layer_backward_fp8(*args), ref.fp8_backward_envelope(*args),
                ref.layer_backward(*args[:8], g=args[8], u=args[9]))

    def compare(got, em, ex, al, what, rounding=None):
        check_close(got, em, 6e-2, al, None, what + " vs FP8-emulating oracle", rounding=rounding)
        e_rms = np.sqrt(np.mean((got - em) ** 2)) / np.sqrt(np.mean(em ** 2))
        x_rms = np.sqrt(np.mean((got - ex) ** 2)) / np.sqrt(np.mean(ex ** 2))
        say(f"  {what}: rms err / rms vs emulating oracle {e_rms:.3e}, vs exact {x_rms:.3e}")
        assert e_rms <= 1e-2, what

    counts = np.diff(offsets)
    for e in (0, int(np.argmax(counts)), wl.E - 1):
        toks, slots = fp8_sub.expert_rows(e, offsets, dst_row, src_tok)
        say(f"  expert {e}: {len(toks)} rows, oracle")
        emu, allow, exact = oracle(toks, slots, [e])
        for name in ("dw1", "dw3", "dw2"):
            compare(got_w[name][e], emu[name][0], exact[name][0], allow[name][0], f"{name}[{e}]")
    tok_s = np.sort(np.random.default_rng(7).choice(wl.T, 32, replace=False))
    toks, slots, experts = fp8_sub.token_rows(tok_s, idx)
    say(f"  dX of {len(tok_s)} tokens ({len(toks)} routed rows, {len(experts)} experts), oracle")
    emu, allow, exact = oracle(toks, slots, experts)
    em, ex, al = (fp8_sub.token_sum(d["dx"], tok_s, toks) for d in (emu, exact, allow))
    compare(host(layer.dx)[tok_s], em, ex, al, "dX sampled", rounding=HALF_ULP_BF16 * np.abs(em))


GATHER_CASES = [c + (None,) for c in (CASES[0], CASES[2], CASES[5], CASES[6])] + [
    ("e72", dict(T=200, h=256, h_ffn=256, E=72, k=4), 9, None),
    # pairs beyond a per-expert capacity dropped before the dispatch: fewer
    # kept rows than pairs, and dropped pairs in dst_row
    ("capacity", dict(T=300, h=256, h_ffn=256, E=8, k=2), 10, 60)]


def gather_entry_matches(wl, inp, cap=None):
    """Run the layer (FP8 backward through moe_grouped_swiglu_bwd_fp8_tok),
    then moe_grouped_swiglu_bwd_fp8 on dispatched bf16 copies of w * dY and
    x, and require every output bit-identical (dXp on the kept rows: rows
    past them are written by neither entry)."""
    T, h, hf, E, k = wl.T, wl.h, wl.h_ffn, wl.E, wl.k
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), MOE_FP8_E4M3,
                          backward=True)
    layer = ops.MoELayer(T, h, hf, E, k, MOE_FP8_E4M3, save_for_backward=True)
    xd, dyd = dev_tensor(inp["x"]), dev_tensor(inp["dy"])
    layer.forward(xd, dev_tensor(inp["w_gate"]), torch.from_numpy(inp["bias"]).to(DEV), P, capacity=cap)
    if cap is not None:
        assert int(layer.offsets[E]) < T * k and int((layer.dst_row < 0).sum()) > 0
    layer.backward(dyd, xd, P)   # the layer's own path: the token-gather entry
    R = layer.R
    dyp = torch.empty(R, h, dtype=torch.bfloat16, device=DEV)
    xp = torch.empty(R, h, dtype=torch.bfloat16, device=DEV)
    ops.moe_permute(dyd, MOE_BF16, None, layer.topk_w, T, h, E, k, None, None, layer.dst_row, None,
                    dyp, MOE_BF16, None, None, 0)
    ops.moe_permute(xd, MOE_BF16, None, None, T, h, E, k, None, None, layer.dst_row, None,
                    xp, MOE_BF16, None, None, 0)
    outs = {n: torch.full_like(getattr(layer, n), float("nan")) for n in ("dxp", "dw1", "dw3", "dw2")}
    ws = torch.empty_like(layer.bws)
    ops.moe_grouped_swiglu_bwd_fp8(layer.dyp_q, layer.dyp_s, dyp, xp, layer.h13, P.struct, layer.offsets, R,
                                   outs["dxp"], outs["dw1"], outs["dw3"], outs["dw2"], ws, layer.bws_bytes)
    torch.cuda.synchronize()
    kept = int(layer.offsets[E])
    for n, t in outs.items():
        got = getattr(layer, n)
        if n == "dxp":
            got, t = got[:kept], t[:kept]
        same = torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32))
        assert same, n


@pytest.mark.parametrize("case,over,seed,cap", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_fp8_backward_token_gather_entry_is_bit_identical(case, over, seed, cap):
    """moe_grouped_swiglu_bwd_fp8_tok (w * dY and Xp gathered from dY and x
    where they are quantized) against moe_grouped_swiglu_bwd_fp8 on the
    dispatched bf16 copies of the same values: every output bit-identical."""
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name=case, dtype="fp8", **over)
    gather_entry_matches(wl, moe_synth.gen_all(wl, seed=seed), cap)
