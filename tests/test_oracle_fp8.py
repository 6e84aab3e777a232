"""Pins for the oracle's FP8 (OCP E4M3FN) codec and per-token / per-channel scales.

Pins: torch's CPU ``float8_e4m3fn`` decode of all 256 codes and its cast of
values within +-448 (a library routine), hand-listed boundary codes of the
format, exact midpoints (ties to even) and the saturation rule.
"""
import numpy as np
import pytest
import torch

import moe_synth
from oracle import moe_ref as ref


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = ref.e4m3_decode(codes)
    lib = _torch_decode(codes)
    nan = np.isnan(lib)
    assert nan.sum() == 2 and np.array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], lib[~nan])


def test_boundary_codes():
    dec = ref.e4m3_decode
    assert dec(np.uint8(0x7E)) == 448.0
    assert dec(np.uint8(0x01)) == 2.0 ** -9          # smallest subnormal
    assert dec(np.uint8(0x07)) == 7 * 2.0 ** -9      # largest subnormal
    assert dec(np.uint8(0x08)) == 2.0 ** -6          # smallest normal
    assert dec(np.uint8(0x38)) == 1.0
    assert dec(np.uint8(0xB8)) == -1.0


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(ref.e4m3_encode(ref.e4m3_decode(codes)), codes)


def test_encode_matches_torch_within_range():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-13, np.log2(448.0), 200000))
    v = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    np.testing.assert_array_equal(ref.e4m3_encode(v), _torch_encode(v))


def test_midpoints_round_to_even():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = ref.e4m3_decode(codes); hi = ref.e4m3_decode(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)    # midpoints are exact in fp32
    got = ref.e4m3_encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    np.testing.assert_array_equal(got, want.astype(np.uint8))
    np.testing.assert_array_equal(got, _torch_encode(mid))


def test_saturation():
    v = np.array([448.0, 449.0, 463.99, 464.0, 1e6, np.float32(3e38)], np.float32)
    assert ref.e4m3_encode(v).tolist() == [0x7E] * 6
    assert ref.e4m3_encode(-v).tolist() == [0xFE] * 6


def test_row_and_column_scales():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 40)).astype(np.float32)
    x[3] = 0
    q, s = ref.quantize_rows(x)
    assert s.dtype == np.float32 and s[3] == 1.0 and np.all(q[3] == 0)
    for r in (0, 1, 2, 4, 5):
        c = int(np.argmax(np.abs(x[r])))
        assert q[r, c] in (0x7E, 0xFE)
        assert s[r] == np.float32(np.abs(x[r]).max() / np.float32(448.0))
    err = np.abs(ref.e4m3_decode(q) * s[:, None] - x)
    assert np.all(err <= np.abs(x) * 2 ** -4 + s[:, None] * 2.0 ** -10)
    w = rng.standard_normal((40, 7)).astype(np.float32)
    qw, sw = ref.quantize_cols(w)
    np.testing.assert_array_equal(qw.T, ref.quantize_rows(w.T)[0])
    np.testing.assert_array_equal(sw, ref.quantize_rows(w.T)[1])


def test_fp8_layer_close_to_exact_layer():
    wl = moe_synth.WORKLOADS["tiny"].scaled(k=1)
    inp = moe_synth.gen_all(wl, seed=3)
    args = (inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], wl.k)
    exact = ref.layer_forward(*args)["y"]
    q = ref.layer_forward_fp8(*args)
    rms = np.sqrt(np.mean(exact ** 2))
    err = q["y"] - exact
    # three E4M3 roundings (x, weights, SwiGLU output) of about 2^-4 relative
    # each: the layer error is a few percent of rms, and not zero
    assert 1e-3 * rms < np.sqrt(np.mean(err ** 2)) < 0.1 * rms
    yt = ref.layer_forward_fp8_tokens(inp["x"], q["idx"], q["w"], inp["w1"], inp["w3"], inp["w2"])
    np.testing.assert_allclose(q["y"], yt, rtol=1e-12, atol=1e-12 * rms)
    cols = np.array([3, 17, 100, 255])
    yc = ref.layer_forward_fp8_tokens(inp["x"], q["idx"], q["w"], inp["w1"], inp["w3"], inp["w2"], cols=cols)
    np.testing.assert_allclose(yc, q["y"][:, cols], rtol=1e-12, atol=1e-12 * rms)


def _bwd_setup(seed, T=9, h=16, hf=12, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = ref.round_bf16(rng.standard_normal((T, h)))
    wg = rng.standard_normal((h, E))
    w1 = ref.round_bf16(rng.standard_normal((E, h, hf)) / np.sqrt(h))
    w3 = ref.round_bf16(rng.standard_normal((E, h, hf)) / np.sqrt(h))
    w2 = ref.round_bf16(rng.standard_normal((E, hf, h)) / np.sqrt(hf))
    dy = ref.round_bf16(rng.standard_normal((T, h)))
    fw = ref.layer_forward(x, wg, None, w1, w3, w2, k)
    return x, dy, w1, w3, w2, fw


def test_fp8_backward_data_flow_equals_bf16_storage_backward():
    """With every quantizer the identity the FP8 backward is the BF16-storage
    backward: same operands, scales and transposes."""
    x, dy, w1, w3, w2, fw = _bwd_setup(0)
    a = ref.layer_backward_fp8(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, fw["g"], fw["u"],
                               quant=False)
    b = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, g=fw["g"], u=fw["u"],
                           bf16_operands=True)
    for key in ("dx", "dw1", "dw3", "dw2"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-12 * np.abs(b[key]).max(), err_msg=key)


def test_fp8_backward_close_to_exact():
    """E4M3 keeps 3 mantissa bits (relative rounding <= 2^-4, ~2^-4/sqrt(3)
    rms for uniform rounding): the FP8 gradients' rms error stays a few
    percent of the exact gradients' rms."""
    x, dy, w1, w3, w2, fw = _bwd_setup(1, T=40, h=64, hf=48, E=4, k=2)
    a = ref.layer_backward_fp8(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, fw["g"], fw["u"])
    b = ref.layer_backward(dy, x, fw["w"], fw["dst_row"], fw["offsets"], w1, w3, w2, g=fw["g"], u=fw["u"])
    for key in ("dx", "dw1", "dw3", "dw2"):
        rms = np.sqrt(np.mean(b[key] ** 2))
        err = np.sqrt(np.mean((a[key] - b[key]) ** 2)) / rms
        assert 5e-3 < err < 0.08, (key, err)      # quantization happened, and is bounded


def test_hand_worked_fp8_layer():
    """The oracle reproduces, value for value, a two-token FP8 layer worked
    out by hand (tests/golden/fp8_hand_case.json): per-token x scales on the
    rows, per-output-channel weight scales on the columns, A's per-row scale
    from its exact value, an E4M3 round-up (280 -> 288) and a tie rounded to
    the even code (168 -> 160)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp8_hand_case.json")) as fh:
        g = json.load(fh)
    arr = lambda k: np.array(g[k], np.float64)
    x = arr("x").astype(np.float32)
    w1, w3, w2 = (arr(k)[None].astype(np.float32) for k in ("w1", "w3", "w2"))
    T = x.shape[0]
    r = ref.layer_forward_fp8(x, np.zeros((x.shape[1], 1), np.float32), None, w1, w3, w2, 1,
                              logits=np.zeros((T, 1), np.float32))
    np.testing.assert_array_equal(r["sx"], arr("x_scale"))
    np.testing.assert_array_equal(r["qx"], np.array(g["x_codes"], np.uint8))
    np.testing.assert_array_equal(r["g"], arr("g"))
    np.testing.assert_array_equal(r["u"], arr("u"))
    np.testing.assert_array_equal(r["a"], arr("a"))
    np.testing.assert_array_equal(r["sa"], arr("a_scale"))
    np.testing.assert_array_equal(r["qa"], np.array(g["a_codes"], np.uint8))
    np.testing.assert_array_equal(r["yp"], arr("yp"))
    np.testing.assert_array_equal(r["y"], arr("y"))
    # the codes decode to the values the derivation names
    np.testing.assert_array_equal(ref.e4m3_decode(r["qa"]), [[448, 288], [-448, 160]])


def test_fp8_backward_subproblems_equal_the_whole_layer():
    """The full-size FP8 backward test hands the oracle sub-problems (one
    expert's routed rows; the routed rows of sampled tokens, each as a token
    of its own).  Pin that premise: on a small layer, the sub-problems give
    the whole-layer oracle's dW1, dW3, dW2 of that expert and dX of those
    tokens, and the same envelope, up to the fp64 summation order."""
    import fp8_sub
    from moe_synth import to_f32
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="sub", dtype="fp8", T=240, h=128, h_ffn=192, E=6, k=3)
    inp = moe_synth.gen_all(wl, seed=11)
    f = lambda key: to_f32(inp[key])
    fw = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    g, u = ref.round_bf16(fw["g"]), ref.round_bf16(fw["u"])
    W = [f("w1"), f("w3"), f("w2")]
    whole = (f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], *W, g, u)
    emu, env = ref.layer_backward_fp8(*whole), ref.fp8_backward_envelope(*whole)
    _, _, _, src_tok = ref.build_index(fw["idx"], wl.E)
    for e in range(wl.E):
        toks, slots = fp8_sub.expert_rows(e, fw["offsets"], fw["dst_row"], src_tok)
        args = fp8_sub.subproblem(f("dy"), f("x"), fw["w"], fw["idx"], fw["dst_row"], g, u, *W, toks, slots, [e])
        se, sv = ref.layer_backward_fp8(*args), ref.fp8_backward_envelope(*args)
        for name in ("dw1", "dw3", "dw2"):
            np.testing.assert_allclose(se[name][0], emu[name][e], rtol=1e-12, atol=1e-12 * np.abs(emu[name]).max())
            np.testing.assert_allclose(sv[name][0], env[name][e], rtol=1e-9, atol=1e-12 * np.abs(env[name]).max())
    tok_s = np.array([0, 5, 17, 100, 239])
    toks, slots, experts = fp8_sub.token_rows(tok_s, fw["idx"])
    args = fp8_sub.subproblem(f("dy"), f("x"), fw["w"], fw["idx"], fw["dst_row"], g, u, *W, toks, slots, experts)
    se, sv = ref.layer_backward_fp8(*args), ref.fp8_backward_envelope(*args)
    np.testing.assert_allclose(fp8_sub.token_sum(se["dx"], tok_s, toks), emu["dx"][tok_s], rtol=1e-12,
                               atol=1e-12 * np.abs(emu["dx"]).max())
    np.testing.assert_allclose(fp8_sub.token_sum(sv["dx"], tok_s, toks), env["dx"][tok_s], rtol=1e-9,
                               atol=1e-12 * np.abs(env["dx"]).max())
