"""GPU parity: every step of the HIP path against the CPU oracle.

Bars: routing ids, counts, offsets, dst_row, src_tok and the dispatch copies
bit-exact (given identical fp32 logits); gate weights within 1e-6 relative;
end-to-end outputs within 2e-2 * rms(ref) (bf16) on tokens whose k-th vs
(k+1)-th logit margin exceeds 1e-3; FP8 within 6e-2 * rms(ref) of the
quantization-emulating oracle.

The rms bars bound the arithmetic.  The expert outputs Yp are kept in fp32;
when y itself is bf16, its own rounding to nearest (at most 2^-8 of its
magnitude) is allowed per element (``y_rounding``): outputs reach 5x rms, and
rounding such a value to bf16 alone moves it by ~2e-2 * rms.  Every check
also counts the elements whose pass needed an allowance (plain error above
the bar) and fails when more than a stated small fraction did, so that a
misplaced row cannot hide inside an allowance.
"""
import os
import sys

import numpy as np
import pytest
import torch

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16, MOE_F32, MOE_FP8_E4M3

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(a):
    """Storage-form numpy (fp32 or bf16 bits) -> device tensor of that type."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


HALF_ULP_BF16 = 2.0 ** -8


def y_rounding(y):
    """Half a bf16 ulp of each output value: its own rounding to bf16."""
    return HALF_ULP_BF16 * np.abs(y)


# At most this fraction of a check's elements may need its allowance (plain
# |err| above the bar).  A misplaced or dropped routed row moves every one of
# its token's h outputs by about rms(ref), far outside any allowance here,
# and is 1/T of the elements or more; the values whose own bf16 rounding or
# quantization boundary the allowances cover are rare (|y| > ~4 rms, or an
# FP8 code at a rounding tie).
MAX_NEED = 1e-3


def check_close(got, want, frac, allowance=None, mask=None, what="", max_need=MAX_NEED, rounding=None):
    """max(|got - want| - rounding - allowance) <= frac * rms(want), where
    ``rounding`` is the output's own rounding to its storage type (allowed
    everywhere) and ``allowance`` any other per-element allowance; at most a
    fraction ``max_need`` of the elements may have |got - want| - rounding
    above frac * rms(want) (they passed only through the allowance).  Prints
    the plain max and rms errors.  Returns the worst ratio."""
    if mask is not None:
        got, want = got[mask], want[mask]
        allowance = None if allowance is None else allowance[mask]
        rounding = None if rounding is None else rounding[mask]
    rms = np.sqrt(np.mean(np.square(want, dtype=np.float64)))
    err = np.abs(got.astype(np.float64) - want)
    err_r = err - (0 if rounding is None else rounding)
    excess = err_r - (0 if allowance is None else allowance)
    if rms == 0:
        # an all-zero reference (e.g. the router gradient with one expert) is matched exactly
        say(f"  {what}: reference is zero; max|got| = {np.abs(got).max():.3e}")
        assert not np.any(got), what
        return 0.0
    worst = excess.max() / rms
    need = int(np.count_nonzero(err_r > frac * rms))
    say(f"  {what}: (max|err| - allowance)/rms = {worst:.3e} (bar {frac:g}); plain max|err|/rms = "
        f"{err.max() / rms:.3e}, rms err/rms = {np.sqrt(np.mean(err ** 2)) / rms:.3e}; "
        f"{need} of {err.size} elements needed the allowance")
    assert worst <= frac, what
    assert need <= max_need * err.size, f"{what}: {need} of {err.size} elements needed the allowance"
    return worst


def check_rms(got, want, frac, what=""):
    """rms(got - want) <= frac * rms(want)."""
    rms = np.sqrt(np.mean(np.square(want, dtype=np.float64)))
    r = np.sqrt(np.mean(np.square(got.astype(np.float64) - want))) / rms
    say(f"  {what}: rms err/rms = {r:.3e} (bar {frac:g})")
    assert r <= frac, what
    return r


def rel_err(got, want, mask=None):
    if mask is not None:
        got, want = got[mask], want[mask]
    rms = np.sqrt(np.mean(np.square(want, dtype=np.float64)))
    return np.abs(got.astype(np.float64) - want).max() / rms


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (300, 8, 2), (1000, 64, 6), (513, 32, 3), (257, 16, 1),
                                   (64, 256, 16), (5, 3, 3)])
def test_route_logits_mode_bit_exact(T, E, k):
    say(f"route logits-mode T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[::7, 1:] = L[::7, :1]                      # exact ties on some rows
    L[::5, 2 % E] = L[::5, 0]
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ops.moe_route(None, None, None, torch.from_numpy(L).to(DEV), T, 0, E, k, MOE_F32, idx, w)
    ri, rw = ref.topk_softmax(L, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)
    if k == 1:
        assert np.all(w.cpu().numpy() == 1.0)


@pytest.mark.parametrize("name,T", [("tiny", 256), ("mixtral", 700), ("dsmoe", 1100), ("m352b_zipf", 513),
                                    ("hunyuan_fp8", 300)])
def test_route_from_x(name, T):
    wl = moe_synth.WORKLOADS[name].scaled(T=T)
    say(f"route gemm {name} T={T}")
    x = moe_synth.gen_tokens(wl, "x", seed=1)
    wg, bias = moe_synth.gen_router(wl, seed=1)
    logits = torch.empty(T, wl.E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, wl.k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, wl.k, dtype=torch.float32, device=DEV)
    xd = dev_tensor(x)
    ops.moe_route(xd, dev_tensor(wg), torch.from_numpy(bias).to(DEV), logits, T, wl.h, wl.E, wl.k,
                  ops.dtype_code(xd), idx, w)
    rl = ref.router_logits(to_f32(x), to_f32(wg), bias)
    gl = logits.cpu().numpy()
    scale = np.sqrt(np.mean(rl.astype(np.float64) ** 2))
    assert np.abs(gl - rl).max() <= 1e-5 * scale + 1e-6
    ri, rw = ref.topk_softmax(rl, wl.k)
    keep = ref.topk_margin(rl, wl.k) > 1e-3
    assert keep.mean() > 0.9
    np.testing.assert_array_equal(idx.cpu().numpy()[keep], ri[keep])
    np.testing.assert_allclose(w.cpu().numpy()[keep], rw[keep], rtol=2e-5)


@pytest.mark.parametrize("T,h,E,k", [(300, 256, 8, 2), (257, 512, 64, 6), (130, 192, 100, 4),
                                     (96, 1024, 16, 1), (64, 128, 256, 16), (200, 384, 24, 3),
                                     (150, 640, 40, 5), (97, 1152, 56, 4)])
def test_route_from_x_selection_on_own_logits(T, h, E, k):
    """The BF16 router's top-k and softmax, applied to the logits it wrote,
    equal the oracle's selection on those same logits, element for element.
    Columns of W_g are duplicated so that whole groups of experts tie
    exactly (every column of the gate product runs the same instructions in
    the same order), which exercises the index tie rule; E = 100 takes the
    W_g staging path for E not a multiple of 8; E = 24, 40, 56 have a last
    32-expert block that is partly empty (its columns wrap onto real ones)."""
    say(f"route selection T={T} h={h} E={E} k={k}")
    rng = np.random.default_rng(E * 7 + k)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    wg = (rng.standard_normal((h, E)) * 0.02).astype(np.float32)
    for dst, src in ((3, 0), (5, 0), (E - 1, 1), (E // 2, 2), (E // 2 + 1, 2)):
        if dst < E and src < E and dst != src:
            wg[:, dst] = wg[:, src]
    wg = moe_synth.f32_to_bf16_bits(wg)
    bias = np.zeros(E, np.float32)
    bias[E // 3] = 0.05
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ops.moe_route(dev_tensor(x), dev_tensor(wg), torch.from_numpy(bias).to(DEV), logits, T, h, E, k,
                  MOE_BF16, idx, w)
    gl = logits.cpu().numpy()
    assert (gl[:, 3] == gl[:, 0]).all()                     # the ties are exact
    ri, rw = ref.topk_softmax(gl, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)


# ------------------------------------------------------- index + dispatch

@pytest.mark.parametrize("T,E,k,h,dt", [(300, 8, 2, 64, "bf16"), (1000, 64, 6, 128, "bf16"),
                                        (513, 32, 3, 256, "bf16"), (257, 16, 1, 64, "f32"),
                                        (777, 5, 5, 24, "bf16"), (4096, 8, 2, 8, "bf16")])
def test_index_and_permute_bit_exact(T, E, k, h, dt):
    say(f"permute T={T} E={E} k={k} h={h} {dt}")
    rng = np.random.default_rng(T * 3 + k)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[: T // 3] = np.arange(k, dtype=np.int32)          # a crowded expert block
    x = rng.standard_normal((T, h)).astype(np.float32)
    if dt == "bf16":
        x = moe_synth.f32_to_bf16_bits(x)
    lay = _perm_buffers(T, E, k, h, dt)
    xd = dev_tensor(x)
    ops.moe_permute(xd, ops.dtype_code(xd), torch.from_numpy(idx).to(DEV), None, T, h, E, k,
                    lay["counts"], lay["offsets"], lay["dst_row"], lay["src_tok"], lay["xp"],
                    ops.dtype_code(xd), None, lay["ws"], lay["ws_bytes"])
    counts, offsets, dst_row, src_tok = ref.build_index(idx, E)
    np.testing.assert_array_equal(lay["counts"].cpu().numpy(), counts)
    np.testing.assert_array_equal(lay["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(lay["dst_row"].cpu().numpy(), dst_row)
    np.testing.assert_array_equal(lay["src_tok"].cpu().numpy(), src_tok)
    want = ref.permute(x, dst_row)
    got = lay["xp"].view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else lay["xp"].cpu().numpy()
    np.testing.assert_array_equal(got, want)
    # second call on the same buffers is deterministic
    ops.moe_permute(xd, ops.dtype_code(xd), torch.from_numpy(idx).to(DEV), None, T, h, E, k,
                    lay["counts"], lay["offsets"], lay["dst_row"], lay["src_tok"], lay["xp"],
                    ops.dtype_code(xd), None, lay["ws"], lay["ws_bytes"])
    np.testing.assert_array_equal(lay["dst_row"].cpu().numpy(), dst_row)


def _perm_buffers(T, E, k, h, dt, dst_dtype=None):
    i32 = dict(dtype=torch.int32, device=DEV)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[dst_dtype or dt]
    wsb = ops.moe_permute_workspace_size(T, E, k)
    return dict(counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                dst_row=torch.empty(T, k, **i32), src_tok=torch.full((T * k,), -7, **i32),
                xp=torch.zeros(T * k, h, dtype=tdt, device=DEV),
                ws=torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV), ws_bytes=wsb)


def test_permute_drops_invalid_ids_and_empty_batch():
    T, E, k, h = 10, 4, 2, 16
    idx = np.array([[0, 1]] * 5 + [[2, 9]] * 5, np.int32)  # id 9 is out of range
    x = moe_synth.f32_to_bf16_bits(np.random.default_rng(0).standard_normal((T, h)).astype(np.float32))
    lay = _perm_buffers(T, E, k, h, "bf16")
    ops.moe_permute(dev_tensor(x), MOE_BF16, torch.from_numpy(idx).to(DEV), None, T, h, E, k,
                    lay["counts"], lay["offsets"], lay["dst_row"], lay["src_tok"], lay["xp"],
                    MOE_BF16, None, lay["ws"], lay["ws_bytes"])
    assert lay["counts"].cpu().tolist() == [5, 5, 5, 0]
    assert lay["offsets"].cpu().tolist() == [0, 5, 10, 15, 15]
    assert (lay["dst_row"].cpu().numpy()[5:, 1] == -1).all()
    lay0 = _perm_buffers(1, E, k, h, "bf16")
    lay0["counts"].fill_(5)
    ops.moe_permute(dev_tensor(x), MOE_BF16, torch.from_numpy(idx).to(DEV), None, 0, h, E, k,
                    lay0["counts"], lay0["offsets"], lay0["dst_row"], lay0["src_tok"], lay0["xp"],
                    MOE_BF16, None, lay0["ws"], lay0["ws_bytes"])
    assert lay0["counts"].cpu().tolist() == [0] * E and lay0["offsets"].cpu().tolist() == [0] * (E + 1)


def test_fp8_hardware_encoder_matches_reference():
    """The quantizers' hardware E4M3 conversion agrees with the library's
    bit-level encoder on every finite fp32 of magnitude <= 464, packed in
    pairs and quadruples (moe_fp8_convert_selftest)."""
    n = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ops.moe_fp8_convert_selftest(n)
    torch.cuda.synchronize()
    assert int(n.item()) == 0


@pytest.mark.parametrize("T,E,k,h", [(300, 16, 1, 6400), (129, 8, 2, 256)])
def test_permute_fp8_bit_exact(T, E, k, h):
    say(f"permute fp8 T={T} h={h}")
    rng = np.random.default_rng(7)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    xf = (rng.standard_normal((T, h)) * np.exp(rng.uniform(-8, 8, (T, 1)))).astype(np.float32)
    xf[3] = 0.0
    x = moe_synth.f32_to_bf16_bits(xf)
    lay = _perm_buffers(T, E, k, h, "bf16", "fp8")
    scale = torch.empty(T * k, dtype=torch.float32, device=DEV)
    ops.moe_permute(dev_tensor(x), MOE_BF16, torch.from_numpy(idx).to(DEV), None, T, h, E, k,
                    lay["counts"], lay["offsets"], lay["dst_row"], lay["src_tok"], lay["xp"],
                    MOE_FP8_E4M3, scale, lay["ws"], lay["ws_bytes"])
    q, s = ref.quantize_rows(to_f32(x))
    _, _, dst_row, src_tok = ref.build_index(idx, E)
    np.testing.assert_array_equal(lay["xp"].cpu().numpy(), ref.permute(q, dst_row))
    np.testing.assert_array_equal(scale.cpu().numpy(), s[src_tok])


@pytest.mark.parametrize("T,E,k,h", [(333, 8, 3, 384), (257, 8, 2, 136), (64, 4, 1, 64), (200, 12, 6, 256)])
def test_permute_row_scale_and_combine(T, E, k, h):
    """Both dispatch kernels (one thread per chunk for k <= 4, one wave per
    token above) and both combine splits (two waves per token when the row
    has an even number of 8-element chunks, else one)."""
    say(f"permute row_scale + combine T={T} E={E} k={k} h={h}")
    rng = np.random.default_rng(3 + k)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
    lay = _perm_buffers(T, E, k, h, "bf16")
    wd = torch.from_numpy(w).to(DEV)
    ops.moe_permute(dev_tensor(x), MOE_BF16, torch.from_numpy(idx).to(DEV), wd, T, h, E, k,
                    lay["counts"], lay["offsets"], lay["dst_row"], lay["src_tok"], lay["xp"],
                    MOE_BF16, None, lay["ws"], lay["ws_bytes"])
    _, _, dst_row, _ = ref.build_index(idx, E)
    want = ref.permute(to_f32(x), dst_row, row_scale=w)
    got = host(lay["xp"])
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-30)
    # combine: weighted sum of routed rows (fp32 accumulate), bf16 and fp32 out
    yp = lay["xp"]
    for out_dt, tol in ((MOE_BF16, 2.0 ** -8), (MOE_F32, 1e-6)):
        y = torch.empty(T, h, dtype=torch.bfloat16 if out_dt == MOE_BF16 else torch.float32, device=DEV)
        ops.moe_combine(yp, MOE_BF16, lay["dst_row"], wd, T, h, k, y, out_dt)
        r = ref.combine(host(yp), dst_row, w)
        assert np.all(np.abs(host(y) - r) <= tol * np.abs(r) + 1e-6 * np.abs(r).max())
    # identity experts: combine(permute(x)) with softmax weights returns x
    L = rng.standard_normal((T, E)).astype(np.float32)
    ri, rw = ref.topk_softmax(L, k)
    _, _, dr, _ = ref.build_index(ri, E)
    xp = dev_tensor(moe_synth.f32_to_bf16_bits(ref.permute(to_f32(x), dr).astype(np.float32)))
    y = torch.empty(T, h, dtype=torch.float32, device=DEV)
    ops.moe_combine(xp, MOE_BF16, torch.from_numpy(dr).to(DEV), torch.from_numpy(rw).to(DEV), T, h, k,
                    y, MOE_F32)
    np.testing.assert_allclose(y.cpu().numpy(), to_f32(x), rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_pack_weights(dt):
    E, h, hf = 3, 256, 384
    wl = moe_synth.Workload("p", 8, h, hf, E, 1, "f32" if dt == "f32" else ("fp8" if dt == "fp8" else "bf16"))
    w1, w3, w2 = moe_synth.gen_experts(wl, seed=2)
    code = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}[dt]
    P = ops.PackedWeights(dev_tensor(w1), dev_tensor(w3), dev_tensor(w2), code)
    torch.cuda.synchronize()
    raw13 = P.w13.cpu().numpy()
    raw2 = P.w2.cpu().numpy()
    # packed row p of w13: gate channel when (p // 32) is even, up channel otherwise
    p = np.arange(2 * hf)
    ch = (p // 64) * 32 + p % 32
    is_up = (p // 32) % 2 == 1
    if dt == "fp8":
        q13 = raw13.reshape(E, 2 * hf, h)
        q2 = raw2.reshape(E, h, hf)
        for e in range(E):
            qa, sa = ref.quantize_cols(to_f32(w1[e])); qb, sb = ref.quantize_cols(to_f32(w3[e]))
            qc, sc = ref.quantize_cols(to_f32(w2[e]))
            want = np.where(is_up[:, None], qb.T[ch], qa.T[ch])
            np.testing.assert_array_equal(q13[e], want)
            np.testing.assert_array_equal(P.w13_scale.cpu().numpy()[e], np.where(is_up, sb[ch], sa[ch]))
            np.testing.assert_array_equal(q2[e], qc.T)
            np.testing.assert_array_equal(P.w2_scale.cpu().numpy()[e], sc)
    else:
        npdt = np.float32 if dt == "f32" else np.uint16
        g13 = raw13.view(npdt).reshape(E, 2 * hf, h)
        g2 = raw2.view(npdt).reshape(E, h, hf)
        want = np.where(is_up[None, :, None], np.transpose(w3, (0, 2, 1))[:, ch], np.transpose(w1, (0, 2, 1))[:, ch])
        np.testing.assert_array_equal(g13, want)
        np.testing.assert_array_equal(g2, np.transpose(w2, (0, 2, 1)))


# ---------------------------------------------------------- whole forward

LAYER_CASES = [
    # name, workload overrides, seed
    ("tiny", dict(), 0),
    ("tiny_k1", dict(k=1), 1),
    ("bf16_small", dict(T=300, h=256, h_ffn=384, E=8, k=2, dtype="bf16"), 2),
    ("bf16_tail_n", dict(T=700, h=384, h_ffn=256, E=4, k=2, dtype="bf16"), 3),
    ("bf16_multi_mtile", dict(T=2048, h=512, h_ffn=512, E=4, k=2, dtype="bf16"), 4),
    ("bf16_e64_k6", dict(T=600, h=256, h_ffn=256, E=64, k=6, dtype="bf16"), 5),
    ("bf16_zipf", dict(T=1000, h=256, h_ffn=384, E=32, k=3, dtype="bf16", zipf_s=1.2), 6),
    ("bf16_one_expert", dict(T=333, h=256, h_ffn=256, E=1, k=1, dtype="bf16"), 7),
    # Mixtral-8x22B and Phi-3.5-MoE proportions (h : h_ffn, E, k) at small size
    ("bf16_8x22b_shape", dict(T=600, h=384, h_ffn=1024, E=8, k=2, dtype="bf16"), 8),
    ("bf16_phi35_shape", dict(T=600, h=512, h_ffn=768, E=16, k=2, dtype="bf16"), 9),
]


def _layer_case(over, seed):
    base = moe_synth.WORKLOADS["tiny"]
    wl = base.scaled(name="case", **over)
    return wl, moe_synth.gen_all(wl, seed=seed)


def _run_gpu_layer(wl, inp, logits_in=None, save=False):
    code = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}[wl.dtype]
    P = ops.PackedWeights(dev_tensor(inp["w1"]), dev_tensor(inp["w3"]), dev_tensor(inp["w2"]), code)
    layer = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, code, save_for_backward=save)
    xd = dev_tensor(inp["x"])
    layer.forward(xd, dev_tensor(inp["w_gate"]), torch.from_numpy(inp["bias"]).to(DEV), P,
                  logits_in=None if logits_in is None else torch.from_numpy(logits_in).to(DEV))
    torch.cuda.synchronize()
    return layer, P


@pytest.mark.parametrize("case,over,seed", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_forward(case, over, seed):
    wl, inp = _layer_case(over, seed)
    say(f"layer fwd {case}: {wl}")
    layer, _ = _run_gpu_layer(wl, inp)
    f = lambda k: to_f32(inp[k])
    r = ref.layer_forward(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    keep = ref.topk_margin(r["logits"], wl.k) > 1e-3
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy()[keep], r["idx"][keep])
    np.testing.assert_array_equal(layer.counts.cpu().numpy().sum(), wl.T * wl.k)
    bf = wl.dtype == "bf16"
    check_close(host(layer.y), r["y"], 2e-2, None, keep, "y", rounding=y_rounding(r["y"]) if bf else None)


@pytest.mark.parametrize("case,over,seed", LAYER_CASES[:5], ids=[c[0] for c in LAYER_CASES[:5]])
def test_layer_forward_logits_mode(case, over, seed):
    """Same layer with the oracle's fp32 logits fed in: every token compared."""
    wl, inp = _layer_case(over, seed)
    f = lambda k: to_f32(inp[k])
    r = ref.layer_forward(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    layer, _ = _run_gpu_layer(wl, inp, logits_in=r["logits"])
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), r["idx"])
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), r["dst_row"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), r["offsets"])
    bf = wl.dtype == "bf16"
    say(f"layer logits-mode {case}")
    check_close(host(layer.y), r["y"], 2e-2, None, None, "y", rounding=y_rounding(r["y"]) if bf else None)
    # expert outputs before the combine (fp32), row by row: the plain bar
    R = wl.T * wl.k
    check_close(host(layer.yp)[:R], r["yp"], 2e-2, None, None, "Yp")
    if bf:
        # same layer with an fp32 output: nothing is rounded to bf16 after FC2
        y32 = torch.empty(wl.T, wl.h, dtype=torch.float32, device=DEV)
        ops.moe_combine(layer.yp, MOE_F32, layer.dst_row, layer.topk_w, wl.T, wl.h, wl.k, y32, MOE_F32)
        check_close(y32.cpu().numpy(), r["y"], 2e-2, None, None, "y fp32")


@pytest.mark.parametrize("over,seed", [(dict(T=300, h=256, h_ffn=384, E=8, k=1, dtype="fp8"), 8),
                                       (dict(T=513, h=384, h_ffn=256, E=4, k=2, dtype="fp8"), 9)])
def test_layer_forward_fp8(over, seed):
    wl, inp = _layer_case(over, seed)
    say(f"layer fwd fp8: {wl}")
    f = lambda k: to_f32(inp[k])
    r = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    layer, _ = _run_gpu_layer(wl, inp, logits_in=r["logits"])
    np.testing.assert_array_equal(layer.xp.cpu().numpy()[: wl.T * wl.k], ref.permute(r["qx"], r["dst_row"]))
    check_fp8_forward(layer, wl, r, f)


def test_layer_forward_fp8_hand_case():
    """The FP8 layer worked out by hand (tests/golden/fp8_hand_case.json),
    zero-padded to h = h_ffn = 128.  Every value of it is exact in fp32 as
    well (power-of-two weight scales, SiLU(G) = G in fp32 for G >= 49), so
    the GPU must reproduce it exactly: the dispatched x codes and per-token
    scales, Yp (kept in fp32) value for value, including A's round-up
    (280 -> 288) and its tie to the even code (168 -> 160), and y as Yp
    rounded once to bf16.  The padding stays zero."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp8_hand_case.json")) as fh:
        g = json.load(fh)
    T, h, hf = 2, 128, 128
    x = np.zeros((T, h), np.float32); x[:, :4] = g["x"]
    w1 = np.zeros((1, h, hf), np.float32); w1[0, :4, :2] = g["w1"]
    w3 = np.zeros((1, h, hf), np.float32); w3[0, :4, :2] = g["w3"]
    w2 = np.zeros((1, hf, h), np.float32); w2[0, :2, :4] = g["w2"]
    b = moe_synth.f32_to_bf16_bits
    assert np.array_equal(to_f32(b(x)), x) and np.array_equal(to_f32(b(w1)), w1)
    inp = dict(x=b(x), w1=b(w1), w3=b(w3), w2=b(w2), w_gate=b(np.zeros((h, 1), np.float32)),
               bias=np.zeros(1, np.float32))
    wl = moe_synth.Workload("fp8_hand", T, h, hf, 1, 1, "fp8")
    layer, _ = _run_gpu_layer(wl, inp, logits_in=np.zeros((T, 1), np.float32))
    xq = layer.xp.cpu().numpy()[:T]
    np.testing.assert_array_equal(xq[:, :4], np.array(g["x_codes"], np.uint8))
    assert not xq[:, 4:].any()
    np.testing.assert_array_equal(layer.xp_scale.cpu().numpy()[:T], np.array(g["x_scale"], np.float32))
    yp = layer.yp.cpu().numpy()[:T]
    np.testing.assert_array_equal(yp[:, :4], np.array(g["yp"], np.float32))
    assert not yp[:, 4:].any()
    y = host(layer.y)
    np.testing.assert_array_equal(y[:, :4], ref.round_bf16(np.array(g["y"])))
    assert not y[:, 4:].any()


def check_fp8_forward(layer, wl, r, f):
    """y of the FP8 forward against the quantization-emulating oracle (A
    quantized from its fp64 value): the FP8 bar (6e-2 * rms) once the
    oracle's allowance for fp32 implementations is granted (the GPU forms A
    in fp32 and quantizes it with an fp32 scale and quotient, so a code or a
    row scale may differ where A or the row's amax sits at a rounding
    boundary), plus half a bf16 ulp of y's own rounding, with few elements
    needing the allowance; rms error below 1e-2 * rms."""
    g_err, u_err = ref.fp8_forward_gu_bound(f("x"), r["dst_row"], r["offsets"], f("w1"), f("w3"))
    env = ref.fp8_forward_envelope(r, f("w1"), f("w3"), f("w2"), g_err, u_err,
                                   ref.topk_weight_bound(r["logits"], r["idx"]))
    got = host(layer.y)
    check_close(got, r["y"], 6e-2, env["y"], None, "y fp8", rounding=y_rounding(r["y"]))
    check_rms(got, r["y"], 1e-2, "y fp8")


def test_layer_deterministic():
    wl, inp = _layer_case(dict(T=700, h=256, h_ffn=384, E=8, k=2, dtype="bf16"), 11)
    a, _ = _run_gpu_layer(wl, inp)
    y1 = a.y.clone()
    b, _ = _run_gpu_layer(wl, inp)
    assert torch.equal(y1.view(torch.int16), b.y.view(torch.int16))


# ------------------------------------------- full-size workload, sampled

class _PerExpert:
    """Widens one expert's bf16 weight to fp32 when the oracle asks for it."""

    def __init__(self, a):
        self.a, self.shape = a, a.shape

    def __getitem__(self, e):
        return to_f32(self.a[e])


def _full_size_sampled(name, n_sample=48, seed=0):
    wl = moe_synth.WORKLOADS[name]
    say(f"full-size {name}: generating inputs")
    inp = moe_synth.gen_all(wl, seed=seed)
    code = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}[wl.dtype]
    say(f"full-size {name}: gpu forward")
    layer, P = _run_gpu_layer(wl, inp)
    rng = np.random.default_rng(123)
    toks = np.sort(rng.choice(wl.T, n_sample, replace=False))
    xs = to_f32(inp["x"][toks])
    rl = ref.router_logits(xs, to_f32(inp["w_gate"]), inp["bias"])
    ri, rw = ref.topk_softmax(rl, wl.k)
    keep = ref.topk_margin(rl, wl.k) > 1e-3
    gi = layer.topk_idx.cpu().numpy()[toks]
    np.testing.assert_array_equal(gi[keep], ri[keep])
    counts = layer.counts.cpu().numpy()
    assert counts.sum() == wl.T * wl.k
    say(f"full-size {name}: oracle on {n_sample} tokens, counts min/max {counts.min()}/{counts.max()}")
    fn = ref.layer_forward_tokens if wl.dtype == "bf16" else ref.layer_forward_fp8_tokens
    w1, w3, w2 = (_PerExpert(inp[n]) for n in ("w1", "w3", "w2"))
    y_ref = fn(xs[keep], ri[keep], rw[keep], w1, w3, w2)
    y_gpu = host(layer.y)[toks][keep]
    frac = 2e-2 if wl.dtype == "bf16" else 6e-2
    return check_close(y_gpu, y_ref, frac, None, None, f"full-size {name} y", rounding=y_rounding(y_ref)), layer


@pytest.mark.slow
def test_full_size_mixtral_sampled():
    _full_size_sampled("mixtral")


@pytest.mark.slow
def test_full_size_mixtral22b_sampled():
    _full_size_sampled("mixtral22b", n_sample=24)


@pytest.mark.slow
def test_full_size_phi35_sampled():
    _full_size_sampled("phi35")


@pytest.mark.slow
def test_full_size_352b_zipf_sampled():
    """Skewed routing: the hottest expert gets several times the mean load."""
    _, layer = _full_size_sampled("m352b_zipf", n_sample=24)
    counts = layer.counts.cpu().numpy()
    say(f"  352B counts: max {counts.max()} ({counts.max() / counts.mean():.2f}x mean), min {counts.min()}")
    assert counts.max() > 5 * counts.mean() and counts.min() > 0


@pytest.mark.slow
def test_full_size_hunyuan_fp8_sampled():
    """FP8 layer at full size: tokens of one expert, a subset of output columns."""
    wl = moe_synth.WORKLOADS["hunyuan_fp8"]
    say("full-size hunyuan_fp8: generating inputs")
    inp = moe_synth.gen_all(wl, seed=0)
    layer, _ = _run_gpu_layer(wl, inp)
    x32 = lambda rows: to_f32(inp["x"][rows])
    rl = ref.router_logits(x32(np.arange(wl.T)), to_f32(inp["w_gate"]), inp["bias"])
    ri, rw = ref.topk_softmax(rl, wl.k)
    keep = ref.topk_margin(rl, wl.k) > 1e-3
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy()[keep], ri[keep])
    e = int(ri[0, 0])
    toks = np.nonzero((ri[:, 0] == e) & keep)[0][:12]
    cols = np.sort(np.random.default_rng(1).choice(wl.h, 64, replace=False))
    say(f"full-size hunyuan_fp8: oracle on {len(toks)} tokens of expert {e}, {len(cols)} columns")
    y_ref = ref.layer_forward_fp8_tokens(x32(toks), ri[toks], rw[toks], _PerExpert(inp["w1"]),
                                         _PerExpert(inp["w3"]), _PerExpert(inp["w2"]), cols=cols)
    y_gpu = host(layer.y)[toks][:, cols]
    # k = 1: y is the expert output rounded once to bf16
    check_close(y_gpu, y_ref, 6e-2, None, None, "full-size fp8 y", rounding=y_rounding(y_ref))
