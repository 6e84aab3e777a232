"""Pins for the oracle's allowance of the FP8 backward (`fp8_backward_envelope`).

The allowance claims: every implementation of the FP8 backward recipe whose
values before each rounding lie within the stated distance of the fp64 ones
(fp32 sums, an fp32 SwiGLU derivative, fp32 gate weights, an fp32 forward)
ends within the allowance of `layer_backward_fp8`.  Pinned by
  * brute force of the per-row quantizer's spread on tiny matrices (every
    combination of candidate values enumerated);
  * nearby implementations: every pre-rounding value replaced by a random
    value within its bound (and the gate weights, G and U moved within
    theirs) must stay inside the allowance;
  * a genuine fp32 evaluation (dA summed in float32 in the allowed order
    with the largest error, float32 exponentials and products for the SwiGLU
    terms) must stay inside the allowance;
  * the allowance is not vacuous: small on average, zero where no quantizer
    input can move.
"""
import itertools

import numpy as np
import pytest

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref


def _case(seed, **over):
    sh = dict(T=160, h=128, h_ffn=128, E=4, k=2)
    sh.update(over)
    wl = moe_synth.WORKLOADS["dsmoe"].scaled(name="env", dtype="fp8", **sh)
    inp = moe_synth.gen_all(wl, seed=seed)
    f = lambda key: to_f32(inp[key])
    fw = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)
    args = (f("dy"), f("x"), fw["w"], fw["dst_row"], fw["offsets"], f("w1"), f("w3"), f("w2"), fw["g"], fw["u"])
    return fw, args


def _excess(got, base, allow):
    return {n: float(((np.abs(got[n] - base[n]) - allow[n]) / np.sqrt(np.mean(base[n] ** 2))).max())
            for n in ("dx", "dw1", "dw3", "dw2")}


def test_rowq_spread_brute_force():
    """Every matrix with entries in [lo, hi] (bf16 values; here each entry has
    one or two candidates, the amax too) quantizes within the spread."""
    rng = np.random.default_rng(0)
    checked = 0
    for trial in range(60):
        vo = ref.round_bf16(rng.normal(0, 1, (2, 4)) * rng.choice([1e-3, 1.0, 30.0]))
        # step some entries (the amax included, sometimes) to their bf16 neighbour
        ulp = np.abs(vo) * 2.0 ** -7
        pick = rng.random(vo.shape) < 0.5
        if trial % 3 == 0:
            pick[:, np.argmax(np.abs(vo), axis=1)] = True
        up = rng.random(vo.shape) < 0.5
        lo = np.where(pick & ~up, ref.round_bf16(vo - ulp), vo)
        hi = np.where(pick & up, ref.round_bf16(vo + ulp), vo)
        qo, spread = ref.rowq_spread(vo, lo, hi)
        q, s = ref.quantize_rows(vo)
        np.testing.assert_array_equal(qo, ref.e4m3_decode(q) * s.astype(np.float64)[:, None])
        cands = [sorted({a, b}) for a, b in zip(lo.ravel(), hi.ravel())]
        for combo in itertools.product(*cands):
            m = np.array(combo).reshape(vo.shape)
            qm, sm = ref.quantize_rows(m)
            dq = ref.e4m3_decode(qm) * sm.astype(np.float64)[:, None]
            assert np.all(np.abs(dq - qo) <= spread), trial
            checked += 1
    assert checked > 1000


def test_rowq_spread_is_zero_without_candidates():
    v = ref.round_bf16(np.random.default_rng(1).normal(0, 1, (5, 33)))
    _, spread = ref.rowq_spread(v, v, v)
    assert not spread.any()


@pytest.mark.parametrize("layer", [False, True], ids=["shared_gu", "layer"])
def test_envelope_contains_nearby_implementations(layer):
    fw, args = _case(2, T=240, E=6, k=3)
    dy, x, w, dst_row, offsets, w1, w3, w2, g, u = args
    if layer:
        g_err, u_err = ref.fp8_forward_gu_bound(x, dst_row, offsets, w1, w3)
        w_err = ref.topk_weight_bound(fw["logits"], fw["idx"])
    else:
        g_err = u_err = w_err = None
    env = ref.fp8_backward_envelope(*args, g_err=g_err, u_err=u_err, w_err=w_err)
    base = ref.layer_backward_fp8(*args)
    rec = {}

    def record(name, e, v):
        rec[(name, e)] = np.array(v, copy=True)
        return v

    ref.layer_backward_fp8(*args, noise=record)
    worst = -np.inf
    for trial in range(4):
        rng = np.random.default_rng(10 + trial)

        def noise(name, e, v):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            mask = rng.random(v.shape) < 0.5
            if name in ("dxp", "dw2", "dw13"):       # an fp32 sum of the implementation's own operands
                d = env["d_dxp"][lo:hi] if name == "dxp" else env["d_" + name][e]
                return v + d * rng.uniform(-1, 1, v.shape) * mask
            return rec[(name, e)] + env["d_" + name][lo:hi] * rng.uniform(-1, 1, v.shape) * mask

        w2_ = w if w_err is None else (w + 0.9 * w_err * rng.uniform(-1, 1, w.shape)).astype(np.float32)
        got = ref.layer_backward_fp8(dy, x, w2_, dst_row, offsets, w1, w3, w2, g, u, noise=noise)
        worst = max(worst, max(_excess(got, base, env).values()))
    assert worst <= 0.0, worst


def test_envelope_contains_fp32_evaluation():
    """dA in float32 from the same codes and fp32 scales, summed as the worst
    member of the allowed class does (one product after the other within
    blocks of 64, then block after block: depth 63 + h/64), then the SwiGLU
    terms in float32, as an fp32 kernel would form them."""
    fw, args = _case(3, T=200, h=1024, h_ffn=128, E=4, k=2)
    dy, x, w, dst_row, offsets, w1, w3, w2, g, u = args
    env = ref.fp8_backward_envelope(*args)
    base = ref.layer_backward_fp8(*args)
    T, k = dst_row.shape
    qdy, sdy = ref.quantize_rows(dy)
    qdyp = ref.permute(qdy, dst_row)
    sdyp = np.zeros(T * k, np.float32)
    for j in range(k):
        sdyp[dst_row[:, j]] = np.float32(1) * w[:, j].astype(np.float32) * sdy.astype(np.float32)
    f32 = {}

    def fp32(name, e, v):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if name == "da":
            qw2, sw2 = ref.quantize_rows(w2[e])
            prod = (ref.e4m3_decode(qdyp[lo:hi]).astype(np.float32)[:, None, :]
                    * ref.e4m3_decode(qw2).astype(np.float32)[None, :, :])       # exact in fp32
            blk = prod.reshape(prod.shape[0], prod.shape[1], -1, 64)
            part = np.add.accumulate(blk, axis=3, dtype=np.float32)[..., -1]
            acc = np.add.accumulate(part, axis=2, dtype=np.float32)[:, :, -1]
            f32["da"] = (acc * sdyp[lo:hi, None]) * sw2.astype(np.float32)[None, :]
            return f32["da"].astype(np.float64)
        if name in ("g", "u"):
            f32[name] = ref.round_bf16(v).astype(np.float32)
            return v
        G, U, dA = f32["g"], f32["u"], f32["da"]
        one = np.float32(1)
        sg = one / (one + np.exp(-G))
        if name == "a":
            return ((G * sg) * U).astype(np.float64)
        if name == "dg":
            return (dA * U * sg * (one + G * (one - sg))).astype(np.float64)
        if name == "du":
            return (dA * (G * sg)).astype(np.float64)
        return v

    got = ref.layer_backward_fp8(*args, noise=fp32)
    moved = {n: float(np.abs(got[n] - base[n]).max()) for n in ("dx", "dw1", "dw3", "dw2")}
    assert max(_excess(got, base, env).values()) <= 0.0
    assert max(moved.values()) > 0.0          # the fp32 evaluation did change something


def test_envelope_is_small():
    fw, args = _case(4, T=300, h=256, h_ffn=256, E=4, k=2)
    env = ref.fp8_backward_envelope(*args)
    base = ref.layer_backward_fp8(*args)
    for n, bound in (("dx", 3e-2), ("dw1", 1e-2), ("dw3", 1e-2), ("dw2", 1e-2)):
        rms = np.sqrt(np.mean(base[n] ** 2))
        assert env[n].mean() / rms < bound, n


# ------------------------------------------------------------ forward

def _fwd_case(seed, **sh):
    wl = moe_synth.WORKLOADS["tiny"].scaled(name="fenv", dtype="fp8", **sh)
    inp = moe_synth.gen_all(wl, seed=seed)
    f = lambda key: to_f32(inp[key])
    return wl, inp, f, ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k)


def _fp32_quant(a):
    """An implementation's quantizer of A: fp32 values, fp32 scale
    amax / 448, codes of the fp32 quotient."""
    return ref.quantize_rows(np.asarray(a, np.float32))


def test_forward_rowq_spread_interval_brute_force():
    """Against the exact (fp64) quantization of vo, every fp32 matrix with
    entries at the ends of [lo, hi] or at the fp32 values next to vo,
    quantized in fp32 (scale and quotient), lands within the spread."""
    rng = np.random.default_rng(5)
    checked = 0
    for trial in range(40):
        vo = rng.normal(0, 1, (2, 3)) * rng.choice([1e-3, 1.0, 30.0])
        d = np.abs(vo) * rng.choice([1e-7, 1e-5, 1e-3]) * (rng.random(vo.shape) < 0.6) + np.abs(vo) * 2.0 ** -23
        lo, hi = vo - d, vo + d
        qo, spread = ref.rowq_spread_interval(vo, lo, hi)
        q, s = ref.quantize_rows_exact(vo)
        np.testing.assert_array_equal(qo, ref.e4m3_decode(q) * s[:, None])
        up = lambda v: np.nextafter(np.float32(v), np.float32(np.inf))
        dn = lambda v: np.nextafter(np.float32(v), np.float32(-np.inf))
        cands = [(np.float32(a) if np.float32(a) >= a else up(a), np.float32(b), dn(c) if np.float32(c) > c else np.float32(c))
                 for a, b, c in zip(lo.ravel(), vo.ravel(), hi.ravel())]
        for combo in itertools.product(*cands):
            m = np.array(combo, np.float32).reshape(vo.shape)
            qm, sm = _fp32_quant(m)
            dq = ref.e4m3_decode(qm) * sm.astype(np.float64)[:, None]
            assert np.all(np.abs(dq - qo) <= spread * (1 + 1e-12) + 1e-300), trial
            checked += 1
    assert checked > 5000


def test_forward_rowq_spread_interval_at_a_midpoint():
    """A row whose exact quotient v / s is an E4M3 midpoint (1.1875, between
    the codes of 1.125 and 1.25) with a scale fp32 does not hold (amax 64,
    s = 1/7): the exact quantizer rounds the tie to the even code (1.25); an
    fp32 implementation holding the same values gets the quotient 1.1874999
    and the code of 1.125.  The spread covers that whole code step although
    the value interval has zero width (the fp32 scale and quotient alone)."""
    vo = np.array([[64.0, 1.1875 / 7.0, -0.5]])
    q, s = ref.quantize_rows_exact(vo)
    assert s[0] == 64.0 / 448.0 and ref.e4m3_decode(q)[0, 1] == 1.25
    qm, sm = _fp32_quant(vo)
    assert ref.e4m3_decode(qm)[0, 1] == 1.125
    deq32 = ref.e4m3_decode(qm)[0, 1] * float(sm[0])
    qo, spread = ref.rowq_spread_interval(vo, vo, vo)
    assert abs(deq32 - qo[0, 1]) > 0.12 * float(s[0])
    assert abs(deq32 - qo[0, 1]) <= spread[0, 1]


def test_forward_envelope_contains_nearby_implementations():
    wl, inp, f, fw = _fwd_case(3, T=263, h=256, h_ffn=128, E=9, k=5, zipf_s=1.2)
    g_err, u_err = ref.fp8_forward_gu_bound(f("x"), fw["dst_row"], fw["offsets"], f("w1"), f("w3"))
    w_err = ref.topk_weight_bound(fw["logits"], fw["idx"])
    env = ref.fp8_forward_envelope(fw, f("w1"), f("w3"), f("w2"), g_err, u_err, w_err)
    offs = fw["offsets"]
    rms = np.sqrt(np.mean(fw["y"] ** 2))
    worst = -np.inf
    for trial in range(4):
        rng = np.random.default_rng(30 + trial)

        def noise(name, e, v):
            m = rng.random(np.shape(v)) < 0.5
            if name == "w":
                return (v + 0.9 * w_err * rng.uniform(-1, 1, v.shape) * m).astype(np.float32)
            lo, hi = int(offs[e]), int(offs[e + 1])
            d = {"g": g_err, "u": u_err, "a": env["d_a"], "yp": env["d_yp"]}[name][lo:hi]
            out = v + d * rng.uniform(-1, 1, v.shape) * m
            return out.astype(np.float32).astype(np.float64)     # fp32 values (Yp stored in fp32)

        got = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k,
                                    logits=fw["logits"], noise=noise, quant_a=_fp32_quant)
        worst = max(worst, float(((np.abs(got["y"] - fw["y"]) - env["y"]) / rms).max()))
    assert worst <= 0.0, worst


def test_forward_envelope_contains_fp32_evaluation():
    """FC1 summed in float32 in the worst allowed order (64-product blocks,
    then block after block) and SiLU(G) U in float32."""
    wl, inp, f, fw = _fwd_case(4, T=200, h=512, h_ffn=128, E=4, k=2)
    g_err, u_err = ref.fp8_forward_gu_bound(f("x"), fw["dst_row"], fw["offsets"], f("w1"), f("w3"))
    env = ref.fp8_forward_envelope(fw, f("w1"), f("w3"), f("w2"), g_err, u_err)
    qx, sx = ref.quantize_rows(f("x"))
    qxp = ref.permute(qx, fw["dst_row"])
    sxp = sx[fw["src_tok"]]
    keep = {}

    def fc1(e, wm):
        lo, hi = int(fw["offsets"][e]), int(fw["offsets"][e + 1])
        q, s = ref.quantize_cols(wm)
        prod = (ref.e4m3_decode(qxp[lo:hi]).astype(np.float32)[:, None, :]
                * ref.e4m3_decode(q).astype(np.float32).T[None, :, :])
        blk = prod.reshape(prod.shape[0], prod.shape[1], -1, 64)
        acc = np.add.accumulate(np.add.accumulate(blk, axis=3, dtype=np.float32)[..., -1], axis=2,
                                dtype=np.float32)[:, :, -1]
        return (acc * sxp[lo:hi, None].astype(np.float32)) * s.astype(np.float32)[None, :]

    def fp32(name, e, v):
        if name in ("g", "u"):
            keep[name] = fc1(e, f("w1")[e] if name == "g" else f("w3")[e])
            return keep[name].astype(np.float64)
        if name == "a":
            G, U = keep["g"], keep["u"]
            return ((G / (np.float32(1) + np.exp(-G))) * U).astype(np.float64)
        return v

    got = ref.layer_forward_fp8(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), wl.k,
                                logits=fw["logits"], noise=fp32, quant_a=_fp32_quant)
    rms = np.sqrt(np.mean(fw["y"] ** 2))
    assert np.abs(got["y"] - fw["y"]).max() > 0
    assert float(((np.abs(got["y"] - fw["y"]) - env["y"]) / rms).max()) <= 0.0


def test_forward_envelope_is_small():
    wl, inp, f, fw = _fwd_case(6, T=300, h=256, h_ffn=256, E=8, k=2)
    g_err, u_err = ref.fp8_forward_gu_bound(f("x"), fw["dst_row"], fw["offsets"], f("w1"), f("w3"))
    env = ref.fp8_forward_envelope(fw, f("w1"), f("w3"), f("w2"), g_err, u_err)
    assert env["y"].mean() / np.sqrt(np.mean(fw["y"] ** 2)) < 2e-2


# -------------------------------------------- single terms, pinned alone

def _fast_exp32(x, ulps):
    """exp(x) as a fast fp32 exponential forms it: 2^(fl32(x * log2 e)),
    rounded to fp32 and moved by ``ulps`` units in the last place (the
    hardware exp2 is within one)."""
    t = (np.float32(x) * np.float32(1.4426950408889634)).astype(np.float32)
    e = np.exp2(t.astype(np.float64)).astype(np.float32)
    for _ in range(abs(ulps)):
        e = np.nextafter(e, np.float32(np.inf) if ulps > 0 else np.float32(0))
    return e


def test_swiglu_eval_bound_against_float32():
    """The fp32 SwiGLU terms of both allowances (`swiglu_eval_bound`): A =
    SiLU(G) U, dG = dA U s (1 + G (1 - s)) and dU = dA SiLU(G) evaluated in
    float32 in the kernels' order, with a fast exponential off by up to one
    ulp either way, stay within the bound plus their own final rounding on
    every sample; and on some samples the error exceeds that final rounding
    alone, so the term is needed."""
    rng = np.random.default_rng(41)
    n = 200000
    G = np.concatenate([rng.normal(0, 3, n // 2), rng.uniform(-40, 40, n // 2)]).astype(np.float32)
    U = rng.normal(0, 2, n).astype(np.float32)
    dA = rng.normal(0, 2, n).astype(np.float32)
    g64, u64, d64 = G.astype(np.float64), U.astype(np.float64), dA.astype(np.float64)
    s64 = ref.sigmoid(g64)
    a64, dg64, du64 = g64 * s64 * u64, d64 * u64 * s64 * (1 + g64 * (1 - s64)), d64 * g64 * s64
    ev_a, ev_dg, ev_du = ref.swiglu_eval_bound(np.abs(g64), np.abs(u64), s64, np.abs(g64 * s64), np.abs(d64))
    one = np.float32(1)
    needed = {"a": 0.0, "dg": 0.0, "du": 0.0}
    for ulps in (-1, 0, 1):
        with np.errstate(over="ignore"):
            s = (one / (one + _fast_exp32(-G, ulps))).astype(np.float32)
        a = ((G * s) * U).astype(np.float64)                     # SiLU(G) U
        dg = (dA * U * s * (one + G * (one - s))).astype(np.float64)
        du = (dA * (G * s)).astype(np.float64)
        for name, got, want, ev in (("a", a, a64, ev_a), ("dg", dg, dg64, ev_dg), ("du", du, du64, ev_du)):
            err = np.abs(got - want) - ref.F32_U * np.abs(want)   # less the final rounding
            assert np.all(err <= ev), (name, ulps, float((err - ev).max()))
            needed[name] = max(needed[name], float(err.max()))
    assert all(v > 0 for v in needed.values()), needed


def test_fp32_sum_bound_covers_worst_order_dA():
    """dA = dYp W2^T summed in float32 in the allowed order with the most
    roundings (64-product blocks one after the other, then block after block)
    stays within the dA term of the backward allowance; the term is needed
    (float32 moves dA)."""
    fw, args = _case(7, T=120, h=2048, h_ffn=128, E=2, k=1)
    dy, x, w, dst_row, offsets, w1, w3, w2, g, u = args
    env = ref.fp8_backward_envelope(*args)
    T, k = dst_row.shape
    qdy, sdy = ref.quantize_rows(dy)
    qdyp = ref.permute(qdy, dst_row)
    sdyp = np.zeros(T * k, np.float32)
    for j in range(k):
        sdyp[dst_row[:, j]] = w[:, j].astype(np.float32) * sdy.astype(np.float32)
    worst, moved = -np.inf, 0.0
    for e in range(w1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        qw2, sw2 = ref.quantize_rows(w2[e])
        a = ref.e4m3_decode(qdyp[lo:hi])
        b = ref.e4m3_decode(qw2)
        prod = (a.astype(np.float32)[:, None, :] * b.astype(np.float32)[None, :, :])   # exact in fp32
        blk = prod.reshape(prod.shape[0], prod.shape[1], -1, 64)
        acc = np.add.accumulate(np.add.accumulate(blk, axis=3, dtype=np.float32)[..., -1], axis=2,
                                dtype=np.float32)[:, :, -1]
        da32 = ((acc * sdyp[lo:hi, None]) * sw2.astype(np.float32)[None, :]).astype(np.float64)
        da64 = (a @ b.T) * sdyp[lo:hi, None].astype(np.float64) * sw2.astype(np.float64)[None, :]
        worst = max(worst, float((np.abs(da32 - da64) - env["d_da"][lo:hi]).max()))
        moved = max(moved, float(np.abs(da32 - da64).max()))
    assert worst <= 0.0 and moved > 0.0
