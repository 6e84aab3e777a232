"""CPU oracle of one GPU's MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it; the two meet only through the
seeded generators in ``moe_synth``.

Plain NumPy in fp64, one expert at a time, no blocking or fusion beyond what
each definition states.  Inputs are the exact stored values (bf16 or fp32),
widened to fp64.

Pages cited (by title; sections as they appear on each page):
  [MSR]  "MegaScale-MoE: 大规模通信高效的生产级混合专家模型训练系统"
         (paper review on xllm-io.github.io)
  [MSD]  "MegaScale-MoE: Large-Scale Communication-Efficient Training of
         Mixture-of-Experts Models in Production" (research digest,
         AI training network primer)
  [DMoE] "DisagMoE：通过解耦的 AF-Pipe 并行实现计算与通信重叠的 MoE 训练"

Readings of points the pages leave open (each also recorded in the design
notes): softmax over the k selected logits; ties broken by lower expert index;
SwiGLU = SiLU(x W1) * (x W3) then W2; gate weights applied in the combine;
dropless dispatch ordered by expert then token; FP8 = OCP E4M3FN with
round-to-nearest-even and saturation at +-448, per-token activation scales
amax/448 and per-output-channel weight scales.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Routing.  [DMoE] §2.1 / Fig. 2(a): a trainable gate scores every expert and
# each token goes to its k highest-scoring experts, whose outputs are summed
# with weights.  [MSR] §三, training flow: routing precedes dispatch.
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_gate: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Gate GEMM ``L = x @ W_g (+ b)``.

    The product is formed in fp64 and rounded once to fp32; the bias is then
    added in fp32.  These fp32 logits are what the top-k step consumes.
    """
    L = (np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64)).astype(np.float32)
    if bias is not None:
        L = (L + np.asarray(bias, np.float32)).astype(np.float32)
    return L


def topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their gate weights.

    Experts are ordered by logit (descending), ties by expert index
    (ascending); slot j holds the j-th expert in that order.  The weights are
    the softmax of the k selected logits, computed in fp64, stored fp32.
    Returns ``idx`` int32 ``[T, k]`` and ``w`` fp32 ``[T, k]``.
    """
    L = np.asarray(logits, np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of the negated logits keeps equal logits in index order
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


def topk_weight_bound(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Bound on |w' - w| for the fp32 gate weights w' of any implementation
    that forms the k-logit softmax in fp32 (x_j = L_j - L_max rounded, an
    exponential within (|x| + 4) u/2 relative, an fp32 sum of k terms, one
    division; u = 2^-23), against `topk_softmax`'s w (the exact value rounded
    to fp32, u/2 more): w (2 X + k + 8) u with X = max_j |x_j|."""
    L = np.asarray(logits, np.float32)
    sel = np.take_along_axis(L, np.asarray(idx, np.int64), axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    X = np.abs(sel - sel[:, :1]).max(axis=1, keepdims=True)
    k = sel.shape[1]
    return w * (2.0 * X + k + 8) * 2.0 ** -23


# --------------------------------------------------------------------------
# Dispatch into expert-contiguous rows.  [MSR] §四, adaptive EP: an extra
# local scatter makes each expert's tokens contiguous.  [MSD] §3.3 Diagram C:
# rows are ordered by expert, then by source; on one GPU the source is the
# token index.  No token is dropped.
# --------------------------------------------------------------------------

def build_index(idx: np.ndarray, E: int):
    """Per-expert counts, offsets, and the row each (token, slot) lands in.

    ``counts[e]`` = number of (t, j) with ``idx[t, j] == e``;
    ``offsets`` = exclusive prefix sum of counts (``offsets[E]`` = rows kept);
    ``dst_row[t, j] = offsets[e] + #{t' < t routed to e}``;
    ``src_tok[dst_row[t, j]] = t``.
    A pair whose id lies outside [0, E) is dropped: it is not counted and its
    ``dst_row`` is -1 (the rows of other experts' GPUs, or dropped tokens).
    ``src_tok`` has ``T*k`` entries; those past ``offsets[E]`` are -1.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    nxt = offsets[:-1].copy()
    dst_row = np.full((T, k), -1, dtype=np.int64)
    src_tok = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if not 0 <= e < E:
                continue
            dst_row[t, j] = nxt[e]
            src_tok[nxt[e]] = t
            nxt[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dst_row.astype(np.int32), src_tok.astype(np.int32))


def permute(x: np.ndarray, dst_row: np.ndarray, row_scale: np.ndarray | None = None) -> np.ndarray:
    """``Xp[dst_row[t, j]] = x[t]`` (times ``row_scale[t, j]`` when given)."""
    T, k = dst_row.shape
    out = np.empty((T * k,) + x.shape[1:], dtype=np.float64 if row_scale is not None else x.dtype)
    for j in range(k):
        v = x if row_scale is None else np.asarray(x, np.float64) * np.asarray(row_scale[:, j], np.float64)[:, None]
        out[dst_row[:, j]] = v
    return out


def combine(yp: np.ndarray, dst_row: np.ndarray, w: np.ndarray | None) -> np.ndarray:
    """Weighted un-permute ``y[t] = sum_j w[t, j] * Yp[dst_row[t, j]]`` (fp64).

    [MSR] §三 training flow, token aggregation; [DMoE] §2.1: the selected
    experts' outputs are reduced by a weighted sum.  ``w=None`` means weight 1
    (the transpose of the dispatch copy, used for dX).
    """
    T, k = dst_row.shape
    y = np.zeros((T,) + yp.shape[1:], dtype=np.float64)
    for j in range(k):
        kept = dst_row[:, j] >= 0                  # dropped pairs contribute nothing
        g = np.zeros((T,) + yp.shape[1:], dtype=np.float64)
        g[kept] = np.asarray(yp[dst_row[kept, j]], np.float64)
        y += g if w is None else np.asarray(w[:, j], np.float64)[:, None] * g
    return y


def local_expert_ids(idx: np.ndarray, e_lo: int, e_count: int) -> np.ndarray:
    """One GPU's share of expert parallelism: the ids of experts
    [e_lo, e_lo + e_count) renumbered from 0, every other id -1.

    [MSD] §3.2 (Diagram B: with the all-gather path each GPU scatters the
    gathered tokens to its own experts and drops the rest, then fills its
    partial outputs for the reduce-scatter); [MSR] §四 (adaptive EP
    communication).  With the all-to-all path the same rows arrive ordered by
    (local expert, source rank); when source ranks hold contiguous token
    ranges that is the (expert, token) order of ``build_index``.
    """
    idx = np.asarray(idx)
    inside = (idx >= e_lo) & (idx < e_lo + e_count)
    return np.where(inside, idx - e_lo, -1)


# --------------------------------------------------------------------------
# SwiGLU experts.  [MSR] §三 core formulas: each expert is a SwiGLU FFN with
# three h x h_ffn matrices; [MSR] §四 selective recomputation names the two
# layers FC1 and FC2.  FC1 produces gate G = Xp W1 and up U = Xp W3, the
# activation is SiLU(G) * U, FC2 multiplies by W2.
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), fp64."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def expert_forward(xp, offsets, w1, w3, w2, keep=True, bf16_storage=False):
    """FC1 -> SwiGLU -> FC2 for every expert's contiguous rows (fp64).

    Returns ``yp`` and, when ``keep``, the intermediates ``g, u, a``.  With
    ``bf16_storage`` the value a BF16 layer stores between FC1 and FC2 is
    rounded to bf16 (nearest even): A; Yp stays as computed (the layer keeps
    it in fp32).
    """
    R = xp.shape[0]
    E = len(offsets) - 1
    h = w2.shape[2]
    yp = np.zeros((R, h), dtype=np.float64)
    if keep:
        hf = w1.shape[2]
        g_all = np.zeros((R, hf)); u_all = np.zeros((R, hf)); a_all = np.zeros((R, hf))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xe = np.asarray(xp[lo:hi], np.float64)
        g = xe @ np.asarray(w1[e], np.float64)
        u = xe @ np.asarray(w3[e], np.float64)
        a = silu(g) * u
        if bf16_storage:
            a = round_bf16(a)
        yp[lo:hi] = a @ np.asarray(w2[e], np.float64)
        if keep:
            g_all[lo:hi] = g; u_all[lo:hi] = u; a_all[lo:hi] = a
    if keep:
        return yp, g_all, u_all, a_all
    return yp


def layer_forward(x, w_gate, bias, w1, w3, w2, k, logits=None):
    """The whole forward layer: route, dispatch, experts, combine.

    ``logits`` may be supplied (fp32) to skip the gate GEMM.  Returns a dict
    with every intermediate; ``y`` is fp64 (the caller rounds to its output
    type).
    """
    E = w1.shape[0]
    L = router_logits(x, w_gate, bias) if logits is None else np.asarray(logits, np.float32)
    idx, w = topk_softmax(L, k)
    counts, offsets, dst_row, src_tok = build_index(idx, E)
    xp = permute(x, dst_row)
    yp, g, u, a = expert_forward(xp, offsets, w1, w3, w2)
    y = combine(yp, dst_row, w)
    return dict(logits=L, idx=idx, w=w, counts=counts, offsets=offsets, dst_row=dst_row,
                src_tok=src_tok, xp=xp, g=g, u=u, a=a, yp=yp, y=y)


def layer_forward_tokens(x_rows, idx_rows, w_rows, w1, w3, w2):
    """Per-token form of the layer, without any permutation.

    ``y[t] = sum_j w[t, j] * FFN_{idx[t, j]}(x[t])``.  Works on any subset of
    tokens, so it checks sampled outputs of a full-size run; it streams one
    expert's weights at a time.
    """
    x_rows = np.asarray(x_rows, np.float64)
    n = x_rows.shape[0]
    y = np.zeros((n, np.shape(w2[0])[1]), dtype=np.float64)
    for e in np.unique(idx_rows):
        tt, jj = np.nonzero(idx_rows == e)
        xe = x_rows[tt]
        a = silu(xe @ np.asarray(w1[e], np.float64)) * (xe @ np.asarray(w3[e], np.float64))
        y[tt] += np.asarray(w_rows[tt, jj], np.float64)[:, None] * (a @ np.asarray(w2[e], np.float64))
    return y


# --------------------------------------------------------------------------
# Backward of the expert path (routing held fixed).  [MSR] §四 selective
# activation recomputation: FC2's backward needs its input and the gradient
# of its output, and FC2's input is recomputed rather than stored; FC1's
# input is obtained again rather than kept.  [MSR] §三 parameter update:
# gradients accumulate in FP32.
# --------------------------------------------------------------------------

def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to fp32 (nearest even), then to bf16 (nearest even); fp64 result."""
    b = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32)).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32).astype(np.float64)


def layer_backward(dy, x, w, dst_row, offsets, w1, w3, w2, g=None, u=None, bf16_operands=False):
    """Gradients of ``y`` w.r.t. ``x`` (expert path only) and every expert weight.

    dYp[dst_row[t,j]] = w[t,j] * dY[t]
    dA = dYp W2^T;  dW2_e = A_e^T dYp_e
    s = sigmoid(G); dG = dA * U * s * (1 + G (1 - s));  dU = dA * SiLU(G)
    dXp = dG W1^T + dU W3^T;  dW1_e = Xp_e^T dG_e;  dW3_e = Xp_e^T dU_e
    dX[t] = sum_j dXp[dst_row[t, j]]
    All fp64.  With ``bf16_operands`` every matrix-product operand that a
    BF16 training step holds in BF16 (dYp, the kept G and U, A, dG, dU, and
    dXp before the sum over slots) is rounded to BF16 first; the arithmetic
    stays fp64.  That is the BF16-storage counterpart of the exact result.
    """
    E = w1.shape[0]
    rb = round_bf16 if bf16_operands else (lambda v: np.asarray(v, np.float64))
    xp = permute(np.asarray(x, np.float64), dst_row)
    dyp = rb(permute(np.asarray(dy, np.float64), dst_row, row_scale=w))
    R, h = xp.shape
    dxp = np.zeros((R, h))
    dw1 = np.zeros(w1.shape); dw3 = np.zeros(w3.shape); dw2 = np.zeros(w2.shape)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W1 = np.asarray(w1[e], np.float64); W3 = np.asarray(w3[e], np.float64)
        W2 = np.asarray(w2[e], np.float64)
        xe = xp[lo:hi]
        ge = rb(xe @ W1 if g is None else np.asarray(g[lo:hi], np.float64))
        ue = rb(xe @ W3 if u is None else np.asarray(u[lo:hi], np.float64))
        s = sigmoid(ge)
        a = rb(ge * s * ue)
        dye = dyp[lo:hi]
        da = dye @ W2.T
        dw2[e] = a.T @ dye
        dg = rb(da * ue * s * (1.0 + ge * (1.0 - s)))
        du = rb(da * ge * s)
        dxp[lo:hi] = rb(dg @ W1.T + du @ W3.T)
        dw1[e] = xe.T @ dg
        dw3[e] = xe.T @ du
    dx = combine(dxp, dst_row, None)
    return dict(dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, dxp=dxp, dyp=dyp)


def expert_grads(xe, dye, w1e, w3e, w2e, bf16_operands=False):
    """One expert's gradients from its routed rows.

    ``xe`` are the expert's routed inputs, ``dye`` the gradients of its
    outputs (already weighted).  Returns dW1, dW3, dW2 and dXp for those rows.
    ``bf16_operands`` as in :func:`layer_backward`.
    """
    rb = round_bf16 if bf16_operands else (lambda v: np.asarray(v, np.float64))
    xe = np.asarray(xe, np.float64); dye = rb(dye)
    W1 = np.asarray(w1e, np.float64); W3 = np.asarray(w3e, np.float64); W2 = np.asarray(w2e, np.float64)
    g = rb(xe @ W1)
    u = rb(xe @ W3)
    s = sigmoid(g)
    da = dye @ W2.T
    dg = rb(da * u * s * (1.0 + g * (1.0 - s)))
    du = rb(da * g * s)
    return xe.T @ dg, xe.T @ du, rb(g * s * u).T @ dye, rb(dg @ W1.T + du @ W3.T)


def layer_backward_tokens(dy_rows, x_rows, idx_rows, w_rows, w1, w3, w2, bf16_operands=False):
    """dX for a subset of tokens: sum over their k experts of that expert's
    input gradient at the token's weighted output gradient (per-token form of
    :func:`layer_backward`)."""
    x_rows = np.asarray(x_rows, np.float64)
    dy_rows = np.asarray(dy_rows, np.float64)
    dx = np.zeros_like(x_rows)
    for e in np.unique(idx_rows):
        tt, jj = np.nonzero(idx_rows == e)
        dye = np.asarray(w_rows[tt, jj], np.float64)[:, None] * dy_rows[tt]
        *_, dxe = expert_grads(x_rows[tt], dye, w1[e], w3[e], w2[e], bf16_operands)
        np.add.at(dx, tt, dxe)
    return dx


# --------------------------------------------------------------------------
# FP8 (E4M3) with per-token activation scales.  [MSR] §三 communication
# compression layer and §四 (FP8 training row): per-token scales replace a
# single per-tensor scale because SwiGLU widens the value range.  [MSD] §3.4:
# FP8 traffic carries per-token scales and is summed in FP32.
# --------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN code -> value (fp64).  0x7F / 0xFF are NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Value -> OCP E4M3FN code, round to nearest (ties to even), saturating.

    Magnitudes above 448 map to 448.  The grid spacing is 2^-9 below 2^-6
    (subnormals) and 2^(e-3) in [2^e, 2^(e+1)).  Rounding is done on the
    exact input value (fp32 or fp64 input, evaluated in fp64).
    """
    v = np.asarray(v, np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))      # a = m * 2^e2, m in [0.5, 1)
    e = np.maximum(e2 - 1, -6)                       # exponent of the binade, floored at the subnormal one
    spacing = np.exp2(e - 3.0)
    q = np.round(a / spacing) * spacing              # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    sub = q < 2.0 ** -6
    _, qe2 = np.frexp(np.where(q > 0, q, 1.0))
    qe = qe2 - 1
    man_n = np.round((q / np.exp2(qe) - 1.0) * 8.0).astype(np.int64)
    code_n = ((qe + 7) << 3) | man_n
    code_s = np.round(q / 2.0 ** -9).astype(np.int64)
    code = np.where(sub, code_s, code_n)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def quant_scale(amax) -> np.ndarray:
    """Scale ``amax / 448`` in fp32 (1 where amax is 0)."""
    amax = np.asarray(amax, np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_rows(v: np.ndarray):
    """Per-row (per-token) quantization of fp32 values.

    ``s[r] = amax_c |v[r, c]| / 448`` and ``q = E4M3(v / s)`` with the
    division done in fp32.  Returns codes uint8 and scales fp32.
    """
    v = np.asarray(v, np.float32)
    s = quant_scale(np.max(np.abs(v), axis=-1) if v.shape[-1] else np.zeros(v.shape[:-1]))
    q = e4m3_encode((v / s[..., None]).astype(np.float32))
    return q, s


def quantize_rows_exact(v: np.ndarray):
    """Per-row quantization of exact (fp64) values, for A = SiLU(G) U.

    ``s[r] = amax_c |v[r, c]| / 448`` and ``q = E4M3(v / s)``, both from the
    fp64 values (1 for an all-zero row).  Returns codes uint8 and fp64 scales.
    """
    v = np.asarray(v, np.float64)
    amax = np.max(np.abs(v), axis=-1) if v.shape[-1] else np.zeros(v.shape[:-1])
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return e4m3_encode(v / s[..., None]), s


def quantize_cols(wm: np.ndarray):
    """Per-output-channel quantization of a weight ``[in, out]`` (fp32 values).

    ``s[n] = amax_i |W[i, n]| / 448``; ``q[i, n] = E4M3(W[i, n] / s[n])``.
    """
    wm = np.asarray(wm, np.float32)
    s = quant_scale(np.max(np.abs(wm), axis=0))
    q = e4m3_encode((wm / s[None, :]).astype(np.float32))
    return q, s


def layer_forward_fp8(x, w_gate, bias, w1, w3, w2, k, logits=None, noise=None, quant_a=None):
    """Forward layer with FP8 GEMM inputs (quantization emulated exactly).

    x is quantized per token before the dispatch copy, so each routed row
    keeps its token's scale; W1, W3 per output channel over h, W2 per output
    channel over h_ffn; FC1 result = (q_x . q_w) * s_x * s_w; A is quantized
    per routed row from its fp64 value (scale amax / 448 and the quotient in
    fp64: ``quantize_rows_exact``); FC2 result = (q_a . q_w2) * s_a * s_w2.  ``noise(name, e, v)``, when
    given, replaces each value an implementation computes before rounding or
    quantizing it ("g", "u", "a"; "yp" for FC2's fp32 sum; "w" with e = -1
    for the gate weights), so that a test can evaluate nearby
    implementations; ``quant_a``, when given, replaces A's quantizer (a test
    passes an fp32 one to emulate an implementation).
    """
    nz = noise if noise is not None else (lambda name, e, v: v)
    qa_fn = quantize_rows_exact if quant_a is None else quant_a
    E = w1.shape[0]
    L = router_logits(x, w_gate, bias) if logits is None else np.asarray(logits, np.float32)
    idx, w = topk_softmax(L, k)
    counts, offsets, dst_row, src_tok = build_index(idx, E)
    qx, sx = quantize_rows(x)
    qxp = permute(qx, dst_row)
    sxp = sx[src_tok]
    R = qxp.shape[0]
    h = w2.shape[2]
    yp = np.zeros((R, h))
    a_all = np.zeros((R, w1.shape[2]))
    g_all = np.zeros((R, w1.shape[2])); u_all = np.zeros((R, w1.shape[2]))
    qa_all = np.zeros((R, w1.shape[2]), np.uint8)
    sa_all = np.ones(R, np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        q1, s1 = quantize_cols(w1[e]); q3, s3 = quantize_cols(w3[e]); q2, s2 = quantize_cols(w2[e])
        xe = e4m3_decode(qxp[lo:hi])
        g = nz("g", e, (xe @ e4m3_decode(q1)) * sxp[lo:hi, None].astype(np.float64) * s1[None, :].astype(np.float64))
        u = nz("u", e, (xe @ e4m3_decode(q3)) * sxp[lo:hi, None].astype(np.float64) * s3[None, :].astype(np.float64))
        a = nz("a", e, silu(g) * u)
        qa, sa = qa_fn(a)
        sa = np.asarray(sa, np.float64)
        yp[lo:hi] = nz("yp", e, (e4m3_decode(qa) @ e4m3_decode(q2)) * sa[:, None] * s2[None, :].astype(np.float64))
        a_all[lo:hi] = a; qa_all[lo:hi] = qa; sa_all[lo:hi] = sa
        g_all[lo:hi] = g; u_all[lo:hi] = u
    y = combine(yp, dst_row, nz("w", -1, w))
    return dict(logits=L, idx=idx, w=w, counts=counts, offsets=offsets, dst_row=dst_row,
                src_tok=src_tok, qx=qx, sx=sx, g=g_all, u=u_all, a=a_all, qa=qa_all, sa=sa_all,
                yp=yp, y=y)


def layer_forward_fp8_tokens(x_rows, idx_rows, w_rows, w1, w3, w2, wq_cache=None, cols=None):
    """Per-token form of :func:`layer_forward_fp8` for sampled tokens.

    ``cols`` restricts the output to those columns of y; W2's per-column
    scales are independent, so only those columns of W2 are quantized.
    """
    qx, sx = quantize_rows(x_rows)
    xd = e4m3_decode(qx) * sx[:, None].astype(np.float64)
    n = xd.shape[0]
    y = np.zeros((n, np.shape(w2[0])[1] if cols is None else len(cols)))
    cache = {} if wq_cache is None else wq_cache
    for e in np.unique(idx_rows):
        if e not in cache:
            w2e = w2[e] if cols is None else np.asarray(w2[e])[:, cols]
            cache[e] = (quantize_cols(w1[e]), quantize_cols(w3[e]), quantize_cols(w2e))
        (q1, s1), (q3, s3), (q2, s2) = cache[e]
        tt, jj = np.nonzero(idx_rows == e)
        xe = xd[tt]
        g = (xe @ e4m3_decode(q1)) * s1[None, :].astype(np.float64)
        u = (xe @ e4m3_decode(q3)) * s3[None, :].astype(np.float64)
        a = silu(g) * u
        qa, sa = quantize_rows_exact(a)
        ye = (e4m3_decode(qa) @ e4m3_decode(q2)) * sa[:, None] * s2[None, :].astype(np.float64)
        y[tt] += np.asarray(w_rows[tt, jj], np.float64)[:, None] * ye
    return y


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit per token (inf if k == E)."""
    L = np.sort(np.asarray(logits, np.float64), axis=1)[:, ::-1]
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    return L[:, k - 1] - L[:, k]


# --------------------------------------------------------------------------
# Router backward and the load-balance loss.  [MSR] §三 (MoE layer
# structure): the gating network is trainable, so W_g (and the router bias)
# get gradients through the gate weights of the combine.  [MSD] §3.2 (the
# discussion of Figure 7): load balance uses an auxiliary loss, following
# DeepSeek-V2.  The pages print no formula; the reading taken is
# DeepSeek-V2's expert-level balance loss
#     L_aux = alpha * sum_e f_e * P_e,
#     f_e   = E / (k T) * (number of (token, slot) pairs routed to e),
#     P_e   = (1/T) * sum_t softmax(L_t)_e      (softmax over all E logits),
# with f_e a count (no gradient) and P_e differentiable.  Routing (the top-k
# selection) is piecewise constant in the logits and is held fixed.
# --------------------------------------------------------------------------

def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Softmax over the last axis in fp64 (max subtracted first)."""
    L = np.asarray(logits, np.float64)
    z = np.exp(L - L.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def aux_balance_loss(logits: np.ndarray, idx: np.ndarray, E: int, k: int, alpha: float) -> float:
    """``alpha * sum_e f_e P_e`` for the routing ``idx`` of these logits."""
    T = logits.shape[0]
    counts = np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.float64)
    f = E / (k * T) * counts
    P = softmax_rows(logits).mean(axis=0)
    return float(alpha * np.sum(f * P))


def router_backward(dy, ysel, x, w_gate, logits, idx, w, alpha, counts=None, T_batch=None):
    """Gradients of ``sum_t <dy_t, y_t> + L_aux`` through the router.

    ``ysel[t, j]`` is the output of expert ``idx[t, j]`` for token t (the row
    ``Yp[dst_row[t, j]]``).  With ``y_t = sum_j w_tj ysel[t, j]`` and
    ``w_t = softmax(L_t[idx_t])``:
        dw[t, j]       = <dy_t, ysel[t, j]>
        dL[t, idx_tj] += w_tj (dw_tj - sum_i w_ti dw_ti)       (top-k softmax)
        dL[t, e]      += s_te (g_e - sum_e' s_te' g_e')        (aux loss)
    with s_t = softmax(L_t) over all experts and g_e = alpha f_e / T.  Then
    dW_g = x^T dL, the router's share of dX is dL W_g^T, and d(bias) = sum_t dL.
    ``counts`` / ``T_batch``: the batch's expert counts and token count, when
    the rows given are a subset of the batch (default: these rows are the
    batch).  Returns a dict with dw, dL, dw_gate, dx, dbias (fp64)."""
    dy = np.asarray(dy, np.float64)
    ysel = np.asarray(ysel, np.float64)
    x = np.asarray(x, np.float64)
    wg = np.asarray(w_gate, np.float64)
    L = np.asarray(logits, np.float64)
    w = np.asarray(w, np.float64)
    T, E = L.shape
    k = idx.shape[1]
    dw = np.einsum("th,tjh->tj", dy, ysel)
    dL = np.zeros((T, E))
    inner = np.sum(w * dw, axis=1)
    for j in range(k):
        dL[np.arange(T), idx[:, j]] += w[:, j] * (dw[:, j] - inner)
    if alpha != 0.0:
        if counts is None:
            counts = np.bincount(np.asarray(idx).ravel(), minlength=E)
        Tb = T if T_batch is None else T_batch
        g = alpha * (E / (k * Tb) * np.asarray(counts, np.float64)) / Tb
        s = softmax_rows(L)
        dL += s * (g[None, :] - (s @ g)[:, None])
    return {"dw": dw, "dL": dL, "dw_gate": x.T @ dL, "dx": dL @ wg.T, "dbias": dL.sum(axis=0)}


def capacity_drop(idx: np.ndarray, logits: np.ndarray, E: int, group: int, capacity: int) -> np.ndarray:
    """Token dropping by affinity ([MSD] §3.2, the discussion of Figure 7:
    tokens are also dropped on each GPU, following DeepSeek-V2, which drops, on each
    device, the tokens with the lowest affinity until the device's budget is
    met).  A device here is a group of ``group`` consecutive experts (one
    GPU's share; ``group = 1`` is a per-expert capacity).  Among the (t, j)
    pairs routed into a group, the ``capacity`` pairs with the highest
    affinity s = softmax(L_t)[e] (over all E experts) are kept, equal
    affinities in dispatch order (expert, then token); the others get id -1,
    which the dispatch drops.  Gate weights are left as they are."""
    idx = np.asarray(idx)
    T, k = idx.shape
    s = softmax_rows(logits)
    out = idx.copy()
    for g0 in range(0, E, group):
        pairs = [(t, j) for t in range(T) for j in range(k) if g0 <= idx[t, j] < g0 + group]
        pairs.sort(key=lambda p: (-s[p[0], idx[p]], idx[p], p[0]))
        for t, j in pairs[capacity:]:
            out[t, j] = -1
    return out


# --------------------------------------------------------------------------
# FP8 backward.  [MSR] §三 (FP8 training row): per-token quantization instead
# of per-tensor; [MSD] §3.4: FP32 sums of FP8 products, per-token scales.  The
# pages give no recipe for the backward products, so (reading):
#   * activation-gradient products dA = dYp W2^T and dXp = [dG|dU] W13^T:
#     the gradient operand per routed row (per token), the weight per output
#     channel of that product, rank-1 rescale of the fp32 sum;
#   * weight-gradient products dW2 = A^T dYp and dW13 = Xp^T [dG|dU] contract
#     over tokens, where a per-token scale cannot leave the sum: both
#     transposed operands are quantized per channel over the expert's rows,
#     again a rank-1 rescale, fp32 dW;
#   * dY is quantized per token before the dispatch copy, so routed row
#     (t, j) carries the codes of dY_t and the scale w_tj * s_t;
#   * the values a BF16 step stores (dYp for the weight gradient, A, dG|dU,
#     dXp) are bf16 before they are quantized or summed.
# --------------------------------------------------------------------------

def quantize_weight_rows(m: np.ndarray):
    """Per-row quantization of a weight block ``[out, in]`` (one scale per
    output channel over the contracted dimension); codes and fp32 scales."""
    return quantize_rows(np.asarray(m, np.float32))


def layer_backward_fp8(dy, x, w, dst_row, offsets, w1, w3, w2, g, u, quant=True, noise=None):
    """Expert-path gradients with FP8 products (quantization emulated).

    ``g``, ``u`` are the forward's kept G and U (per routed row).  With
    ``quant=False`` every quantizer is the identity (codes = values, scales
    1, and dYp the stored bf16 value): the data flow alone, equal to
    ``layer_backward(bf16_operands=True)`` up to the fp64 summation order.
    ``noise(name, e, v)``, when given, returns a replacement for each value
    that an implementation computes before rounding it (names "g", "u" for the
    kept G, U; "da"; "dg", "du"; "a"; "dxp", "dw2", "dw13" for the fp32 sums)
    so that a test can evaluate nearby implementations.
    Returns dx, dw1, dw3, dw2, dxp."""
    if quant:
        qrows = lambda v: quantize_rows(np.asarray(v, np.float32))
        dec = e4m3_decode
    else:
        qrows = lambda v: (np.asarray(v, np.float64), np.ones(np.shape(v)[0]))
        dec = lambda c: np.asarray(c, np.float64)
    nz = noise if noise is not None else (lambda name, e, v: v)
    E = w1.shape[0]
    T, k = dst_row.shape
    dy = np.asarray(dy, np.float64)
    w = np.asarray(w, np.float64)
    xp = permute(np.asarray(x, np.float64), dst_row)
    R, h = xp.shape
    # dYp as stored in bf16, for the weight gradient
    dyp_b = round_bf16(permute(dy, dst_row, row_scale=w))
    # dYp for the activation gradient: codes of dY_t, scale w_tj * s_t (without
    # quantization: the stored bf16 dYp, as in the BF16 step)
    if quant:
        qdy, sdy = qrows(dy)
        qdyp = permute(qdy, dst_row)
        sdyp = np.ones(R)
        for j in range(k):
            kept = dst_row[:, j] >= 0
            sdyp[dst_row[kept, j]] = np.asarray(w[kept, j], np.float32) * np.asarray(sdy[kept], np.float32)
    else:
        qdyp, sdyp = dyp_b, np.ones(R)
    dxp = np.zeros((R, h))
    dw1 = np.zeros(w1.shape); dw3 = np.zeros(w3.shape); dw2 = np.zeros(w2.shape)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W1 = np.asarray(w1[e], np.float64); W3 = np.asarray(w3[e], np.float64)
        W2 = np.asarray(w2[e], np.float64)
        hf = W1.shape[1]
        # dA = dYp W2^T: B rows are W2's h_ffn rows (contracted over h)
        qw2, sw2 = qrows(W2)
        da = (dec(qdyp[lo:hi]) @ dec(qw2).T) * sdyp[lo:hi, None] * np.asarray(sw2, np.float64)[None, :]
        da = nz("da", e, da)
        ge = round_bf16(nz("g", e, g[lo:hi])); ue = round_bf16(nz("u", e, u[lo:hi]))
        s = sigmoid(ge)
        a = round_bf16(nz("a", e, ge * s * ue))
        dgu = round_bf16(np.concatenate([nz("dg", e, da * ue * s * (1.0 + ge * (1.0 - s))),
                                         nz("du", e, da * ge * s)], axis=1))
        # dXp = [dG|dU] [W1|W3]^T: B rows are the h rows of [W1 | W3]
        w13 = np.concatenate([W1, W3], axis=1)                     # [h, 2hf]
        qgu, sgu = qrows(dgu)
        qw13, sw13 = qrows(w13)
        dxp[lo:hi] = round_bf16(nz("dxp", e, (dec(qgu) @ dec(qw13).T) * np.asarray(sgu, np.float64)[:, None]
                                    * np.asarray(sw13, np.float64)[None, :]))
        # weight gradients: transposed operands per channel over the expert's rows
        qat, sat = qrows(a.T)                                      # [hf, rows]
        qdt, sdt = qrows(dyp_b[lo:hi].T)                           # [h, rows]
        dw2[e] = nz("dw2", e, (dec(qat) @ dec(qdt).T) * np.asarray(sat, np.float64)[:, None]
                    * np.asarray(sdt, np.float64)[None, :])
        qxt, sxt = qrows(xp[lo:hi].T)                              # [h, rows]
        qgt, sgt = qrows(dgu.T)                                    # [2hf, rows]
        dw13 = nz("dw13", e, (dec(qxt) @ dec(qgt).T) * np.asarray(sxt, np.float64)[:, None]
                  * np.asarray(sgt, np.float64)[None, :])
        dw1[e] = dw13[:, :hf]
        dw3[e] = dw13[:, hf:]
    dx = combine(dxp, dst_row, None)
    return dict(dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, dxp=dxp)


# --------------------------------------------------------------------------
# Allowance of the FP8 backward.  A quantizer turns a tiny difference before
# it into a whole code step (up to 1/8 of the value) when the value sits at a
# rounding boundary, and into a new scale for its whole row when the row's
# amax sits at a bf16 rounding boundary.  Every implementation that sums in
# fp32 (any order) and evaluates the SwiGLU derivative in fp32 holds, before
# each bf16 rounding, a value within a proven distance of the fp64 one; the
# envelope below pushes those distances through the roundings, quantizers and
# products, and bounds per output element how far such an implementation's
# result can be from `layer_backward_fp8`'s.
#
# Error bounds used (u = 2^-23 bounds one fp32 rounding, truncating or not):
#   * an fp32 sum whose addition tree has depth D (any order within it) is
#     within gamma(D) * sum|terms| of the exact sum, gamma(D) = D u / (1 - D u)
#     (the standard bound for summation trees); the class allowed here forms
#     partial sums of at most 64 products (D <= 63), adds them one after the
#     other (n/64) and then at most 8 partial results, and rescales (2 more
#     roundings);
#   * with s = 1 / (1 + exp(-G)) evaluated in fp32 (the exponential within
#     (|G| + 4) u/2 relative), dG = dA U s (1 + G (1 - s)) is within
#     6 u (1 + |G|)^2 |dA U s|, and dU = dA SiLU(G), A = SiLU(G) U within
#     4 u (1 + |G|) of their magnitude (SiLU(G) = G s);
#   * where the kept G, U are themselves only known within a span of bf16
#     values, |SiLU'| <= 1.1 and |SiLU''| <= 0.55 bound the change.
# --------------------------------------------------------------------------

F32_U = 2.0 ** -23


def fp32_sum_gamma(n):
    """gamma of an fp32 sum of n terms in the class above: depth
    63 + ceil(n / 64) + 8, plus 2 roundings of the rescale."""
    d = 63 + (n + 63) // 64 + 8 + 2
    return d * F32_U / (1.0 - d * F32_U)


def swiglu_eval_bound(g_abs, u_abs, s, silu_abs, da_abs):
    """Bounds of an fp32 evaluation of the SwiGLU terms, from magnitudes:
    |G|, |U|, s = sigmoid(G), |SiLU(G)| = |G s| and |dA| (upper bounds of
    them where G, U, dA are only known within a span).  The class bounded:
    s = 1 / (1 + exp(-G)) with the exponential within (|G| + 4) u/2
    relative and one rounding per operation, u = 2^-23.  Returns the bounds
      A  = SiLU(G) U:                 4 u (1 + |G|) |SiLU(G)| |U|
      dG = dA U s (1 + G (1 - s)):    6 u (1 + |G|)^2 |dA| |U| s
      dU = dA SiLU(G):                4 u (1 + |G|) |dA| |SiLU(G)|
    (the final rounding of each result to fp32 is not included)."""
    a = 4.0 * F32_U * (1.0 + g_abs) * silu_abs * u_abs
    dg = 6.0 * F32_U * (1.0 + g_abs) ** 2 * da_abs * u_abs * s
    du = 4.0 * F32_U * (1.0 + g_abs) * da_abs * silu_abs
    return a, dg, du


def bf16_span(v, d):
    """Lowest and highest bf16 value that rounding any number within ``d``
    of ``v`` can give (rounding is monotone)."""
    v = np.asarray(v, np.float64)
    return round_bf16(v - d), round_bf16(v + d)


def rowq_spread(vo, lo, hi):
    """Per-row quantization (``quantize_rows``) of the bf16 values ``vo``
    against every matrix with elements in ``[lo, hi]`` (bf16 values, lo <=
    vo <= hi).  Returns the dequantized values of ``vo`` and, per element, a
    bound on the distance to the dequantized value of any such matrix.

    For a fixed scale the quantizer is monotone, so the two ends of an
    element's span decide.  A row's amax can take every bf16 value between
    the largest lower and the largest upper magnitude; where that is one or
    two values, both scales are evaluated at both ends.  Otherwise any
    candidate b is within half an E4M3 step of its dequantized value (|b|/16
    for normal codes, 2^-10 s below 2^-6 s) plus the saturation excess (at
    most the amax's own span)."""
    vo = np.asarray(vo, np.float64)
    q, s = quantize_rows(vo)
    s64 = s.astype(np.float64)[:, None]
    qo = e4m3_decode(q) * s64
    straddle = (lo <= 0) & (hi >= 0)
    m_lo = np.where(straddle, 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    m_hi = np.maximum(np.abs(lo), np.abs(hi))
    a_lo = m_lo.max(axis=1) if vo.shape[1] else np.zeros(vo.shape[0])
    a_hi = m_hi.max(axis=1) if vo.shape[1] else np.zeros(vo.shape[0])
    s_lo = quant_scale(a_lo)[:, None]
    s_hi = quant_scale(a_hi)[:, None]
    bits = lambda a: np.asarray(a, np.float32).view(np.uint32).astype(np.int64) >> 16
    few = ((bits(a_hi) - bits(a_lo) <= 1) & (a_lo > 0))[:, None]

    def deq(b, sc):
        return e4m3_decode(e4m3_encode((np.asarray(b, np.float32) / sc).astype(np.float32))) * sc.astype(np.float64)

    ends = np.maximum(np.abs(deq(lo, s_lo) - qo), np.abs(deq(hi, s_lo) - qo))
    ends = np.maximum(ends, np.maximum(np.abs(deq(lo, s_hi) - qo), np.abs(deq(hi, s_hi) - qo)))
    crude = (np.maximum(np.abs(qo - lo), np.abs(qo - hi)) + m_hi / 16.0
             + 2.0 ** -10 * s_hi.astype(np.float64) + (a_hi - a_lo)[:, None] + 2.0 ** -20 * a_hi[:, None])
    return qo, np.where((s_lo == s_hi) | few, ends, crude)


def product_spread(ao, da, bo, db, n):
    """Bound on |A' B'^T - ao bo^T| for |A' - ao| <= da, |B' - bo| <= db
    elementwise, the product summed in fp32 over n terms and rescaled."""
    aa, ab = np.abs(ao), np.abs(bo)
    return da @ ab.T + aa @ db.T + da @ db.T + fp32_sum_gamma(n + 2) * ((aa + da) @ (ab + db).T)


def fp8_forward_gu_bound(x, dst_row, offsets, w1, w3):
    """Distance bound of an fp32 FC1 (FP8 operands, any summation order) from
    the fp64 G and U of `layer_forward_fp8`, per routed row."""
    qx, sx = quantize_rows(np.asarray(x, np.float32))
    qxp = permute(qx, dst_row)
    sxp = np.zeros(qxp.shape[0])
    T, k = dst_row.shape
    for j in range(k):
        kept = dst_row[:, j] >= 0
        sxp[dst_row[kept, j]] = sx[kept]
    h = qxp.shape[1]
    dg = np.zeros((qxp.shape[0], w1.shape[2])); du = np.zeros_like(dg)
    for e in range(w1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ax = np.abs(e4m3_decode(qxp[lo:hi])) * sxp[lo:hi, None]
        for wm, out in ((w1[e], dg), (w3[e], du)):
            q, s = quantize_cols(wm)
            out[lo:hi] = fp32_sum_gamma(h + 2) * (ax @ (np.abs(e4m3_decode(q)) * s.astype(np.float64)[None, :]))
    return dg, du


def fp8_backward_envelope(dy, x, w, dst_row, offsets, w1, w3, w2, g, u, g_err=None, u_err=None, w_err=None):
    """Per-element allowance of `layer_backward_fp8` (same arguments): a
    bound on |result - layer_backward_fp8(...)| for every implementation
    that follows the same recipe with fp32 sums and an fp32 SwiGLU
    derivative.  ``g_err``, ``u_err``: distance bounds of the implementation's
    G, U before their bf16 rounding (None: it keeps exactly round_bf16(g),
    round_bf16(u)); ``w_err``: bounds of its gate weights' distance from
    ``w`` ([T, k]; None: it uses ``w`` itself).

    Returns the allowances of dx, dw1, dw3, dw2, dxp; the bounds d_g, d_u,
    d_da, d_dg, d_du, d_a (per routed row) on the distance of the values an
    implementation rounds from the fp64 ones; and d_dxp, d_dw2, d_dw13, the
    bounds of each fp32 sum's own rounding error (over its own operands)."""
    E = w1.shape[0]
    T, k = dst_row.shape
    dy = np.asarray(dy, np.float64)
    w = np.asarray(w, np.float64)
    xp = permute(np.asarray(x, np.float64), dst_row)
    R, h = xp.shape
    hf = w1.shape[2]
    # dYp = w dY rounded to bf16: with the weights only known within w_err,
    # any bf16 value in the span; the dA row scale w s_t moves by w_err s_t
    wdy = permute(dy, dst_row, row_scale=w)
    dyp_b = round_bf16(wdy)
    w_err = np.zeros(w.shape) if w_err is None else np.asarray(w_err, np.float64)
    w_rel = permute(np.ones((T, 1)), dst_row, row_scale=w_err / np.maximum(w, 1e-300))[:, 0]
    d_wdy = permute(np.abs(dy), dst_row, row_scale=w_err) + (w_err > 0).any() * F32_U * np.abs(wdy)
    dyp_l, dyp_h = bf16_span(wdy, d_wdy)
    qdy, sdy = quantize_rows(np.asarray(dy, np.float32))
    qdyp = permute(qdy, dst_row)
    sdyp = np.ones(R)
    for j in range(k):
        kept = dst_row[:, j] >= 0
        sdyp[dst_row[kept, j]] = np.asarray(w[kept, j], np.float32) * np.asarray(sdy[kept], np.float32)
    g_err = np.zeros((R, hf)) if g_err is None else np.asarray(g_err, np.float64)
    u_err = np.zeros((R, hf)) if u_err is None else np.asarray(u_err, np.float64)
    out = {n: np.zeros((R, hf)) for n in ("d_da", "d_dg", "d_du", "d_a")}
    out["d_g"], out["d_u"] = g_err, u_err
    out["d_dxp"] = np.zeros((R, h)); out["dxp"] = np.zeros((R, h))
    dxp_abs = np.zeros((R, h))
    for n, shp in (("dw1", w1.shape), ("dw3", w3.shape), ("dw2", w2.shape), ("d_dw2", w2.shape),
                   ("d_dw13", (E, h, 2 * hf))):
        out[n] = np.zeros(shp)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        n_e = hi - lo
        # dA: exact codes, fp32 sum over h
        qw2, sw2 = quantize_rows(np.asarray(w2[e], np.float32))
        adyp = np.abs(e4m3_decode(qdyp[lo:hi])) * sdyp[lo:hi, None]
        aw2 = np.abs(e4m3_decode(qw2)) * sw2.astype(np.float64)[:, None]
        qdyv = e4m3_decode(qdyp[lo:hi]) * sdyp[lo:hi, None]
        da = qdyv @ (e4m3_decode(qw2) * sw2.astype(np.float64)[:, None]).T
        d_da = fp32_sum_gamma(h + 2) * (adyp @ aw2.T)
        d_da = d_da + (w_rel[lo:hi, None] + F32_U * (w_rel[lo:hi, None] > 0)) * (np.abs(da) + d_da)
        # the kept G, U: the bf16 values any such implementation may hold
        gl, gh = bf16_span(g[lo:hi], g_err[lo:hi])
        ul, uh = bf16_span(u[lo:hi], u_err[lo:hi])
        ge, ue = round_bf16(g[lo:hi]), round_bf16(u[lo:hi])
        dG, dU = gh - gl, uh - ul
        umax = np.maximum(np.abs(ul), np.abs(uh))
        s = sigmoid(ge)
        gmax = np.abs(ge) + dG                       # |G'| for every candidate G'
        smax = sigmoid(ge + dG)                      # s(G') <= s(ge + dG)
        silu_max = np.abs(ge * s) + 1.1 * dG
        dabs = np.abs(da) + d_da
        # the fp32 evaluation of the SwiGLU terms, at the spans' largest magnitudes
        ev_a, ev_dg, ev_du = swiglu_eval_bound(gmax, umax, smax, silu_max, dabs)
        # A = SiLU(G) U before its bf16 rounding
        a0 = ge * s * ue
        d_a = 1.1 * dG * umax + np.abs(ge * s) * dU + ev_a
        # dG, dU before their bf16 rounding
        fgo = ue * s * (1.0 + ge * (1.0 - s))
        d_dg = d_da * np.abs(fgo) + dabs * (1.1 * dU + 0.55 * umax * dG) + ev_dg
        d_du = d_da * np.abs(ge * s) + dabs * 1.1 * dG + ev_du
        dg0, du0 = da * fgo, da * ge * s
        for n, v in (("d_da", d_da), ("d_dg", d_dg), ("d_du", d_du), ("d_a", d_a)):
            out[n][lo:hi] = v
        a_o = round_bf16(a0)
        a_l, a_h = bf16_span(a0, d_a)
        gu0 = np.concatenate([dg0, du0], axis=1)
        d_gu = np.concatenate([d_dg, d_du], axis=1)
        gu_o = round_bf16(gu0)
        gu_l, gu_h = bf16_span(gu0, d_gu)
        # dXp = [dG|dU] W13^T: per-row codes of dG|dU, exact weight codes
        qgu, sp_gu = rowq_spread(gu_o, gu_l, gu_h)
        w13 = np.concatenate([np.asarray(w1[e], np.float64), np.asarray(w3[e], np.float64)], axis=1)
        q13, s13 = quantize_rows(np.asarray(w13, np.float32))
        b13 = e4m3_decode(q13) * s13.astype(np.float64)[:, None]
        c = qgu @ b13.T
        d_c = product_spread(qgu, sp_gu, b13, np.zeros_like(b13), 2 * hf)
        out["d_dxp"][lo:hi] = fp32_sum_gamma(2 * hf + 2) * ((np.abs(qgu) + sp_gu) @ np.abs(b13).T)
        # the stored bf16 dXp: any value between the roundings of the span's ends
        c_o = round_bf16(c)
        c_l, c_h = bf16_span(c, d_c)
        out["dxp"][lo:hi] = np.maximum(c_h - c_o, c_o - c_l)
        dxp_abs[lo:hi] = np.abs(c_o)
        # dW2 = A^T dYp: A^T per channel (span), dYp^T exact
        qat, sp_at = rowq_spread(a_o.T, a_l.T, a_h.T)
        qdt, sp_dt = rowq_spread(dyp_b[lo:hi].T, dyp_l[lo:hi].T, dyp_h[lo:hi].T)
        out["dw2"][e] = product_spread(qat, sp_at, qdt, sp_dt, n_e)
        out["d_dw2"][e] = fp32_sum_gamma(n_e + 2) * ((np.abs(qat) + sp_at) @ np.abs(qdt).T)
        # dW13 = Xp^T [dG|dU]: Xp^T exact, [dG|dU]^T per channel (span)
        qxt, sp_xt = rowq_spread(xp[lo:hi].T, xp[lo:hi].T, xp[lo:hi].T)
        qgt, sp_gt = rowq_spread(gu_o.T, gu_l.T, gu_h.T)
        d13 = product_spread(qxt, sp_xt, qgt, sp_gt, n_e)
        out["d_dw13"][e] = fp32_sum_gamma(n_e + 2) * (np.abs(qxt) @ (np.abs(qgt) + sp_gt).T)
        out["dw1"][e] = d13[:, :hf]
        out["dw3"][e] = d13[:, hf:]
    # dX: the k stored rows of a token added in fp32 and rounded to bf16 once;
    # that rounding of the result itself (half a bf16 ulp) is left to the caller
    mag = combine(dxp_abs + out["dxp"], dst_row, None)
    out["dx"] = combine(out["dxp"], dst_row, None) + fp32_sum_gamma(k) * mag + 2.0 ** -8 * combine(out["dxp"], dst_row, None)
    return out


# --------------------------------------------------------------------------
# Allowance of the FP8 forward.  The oracle quantizes A = SiLU(G) U per
# routed row from its fp64 value; an implementation forms A in fp32 from an
# fp32 FC1, takes the row's amax of that, rounds amax / 448 to an fp32 scale
# and encodes the fp32 quotient.  Where an A value or the row's amax sits at a
# rounding boundary the two choose different codes or scales, and the
# allowance below bounds, per output element, how far any such implementation
# can be from `layer_forward_fp8`.  For a fixed scale the code is monotone in
# the value, and for a fixed code the dequantized value is monotone in the
# scale, so the ends of the value and scale intervals decide.
# --------------------------------------------------------------------------

def rowq_spread_interval(vo, lo, hi):
    """``quantize_rows_exact`` of the fp64 values ``vo`` against the per-row
    quantization of any matrix A' with entries in [lo, hi] (lo <= vo <= hi)
    whose scale is amax(|A'|) / 448 rounded to fp32 and whose codes are those
    of the fp32 quotients (each within 2^-24 relative of the exact one).
    Returns the oracle's dequantized values and a per-element bound on the
    distance to the dequantized values of any such A'."""
    vo = np.asarray(vo, np.float64)
    q, s = quantize_rows_exact(vo)
    qo = e4m3_decode(q) * s[:, None]
    lo = np.asarray(lo, np.float64); hi = np.asarray(hi, np.float64)
    straddle = (lo <= 0) & (hi >= 0)
    m_lo = np.where(straddle, 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    m_hi = np.maximum(np.abs(lo), np.abs(hi))
    r = 2.0 ** -24                                    # one fp32 rounding, relative
    a_lo = m_lo.max(axis=1) if vo.shape[1] else np.zeros(vo.shape[0])
    a_hi = m_hi.max(axis=1) if vo.shape[1] else np.zeros(vo.shape[0])
    s_lo = (a_lo / E4M3_MAX * (1 - r))[:, None]
    s_hi = (a_hi / E4M3_MAX * (1 + r))[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        lower = e4m3_decode(e4m3_encode(m_lo / s_hi * (1 - r))) * s_lo
        upper = e4m3_decode(e4m3_encode(np.where(s_lo > 0, m_hi / s_lo * (1 + r), E4M3_MAX))) * s_hi
    aq = np.abs(qo)
    spread = np.where(straddle, aq + upper, np.maximum(aq - lower, upper - aq))
    # a row that may be all zero (amax interval reaching 0): any scale, every
    # dequantized magnitude at most amax(|A'|) * (1 + 1/16) (saturation aside)
    crude = aq + m_hi.max(axis=1, initial=0.0)[:, None] * (1 + 2.0 ** -4) * (1 + 4 * r)
    return qo, np.maximum(np.where(a_lo[:, None] > 0, spread, crude), 0.0)


def fp8_forward_envelope(fw, w1, w3, w2, g_err=None, u_err=None, w_err=None):
    """Per-element allowance of `layer_forward_fp8` (its result ``fw``): a
    bound on |y - fw["y"]| for every implementation with an fp32 FC1 (G, U
    within ``g_err`` / ``u_err`` of fw's), A = SiLU(G) U in fp32, the row
    quantization of that fp32 A (fp32 scale and quotient), FC2 summed in fp32
    (trees as for the backward) and stored in fp32, and gate weights within
    ``w_err``, added in fp32 and the sum rounded once (the rounding of the
    result itself, half a bf16 ulp of y, is left to the caller; the rounding
    of the allowance is included).  Returns y, yp (the stored Yp against
    fw's), and the bounds d_a (A before quantization, fp32 evaluation only,
    per routed row) and d_yp (FC2's own fp32 sum)."""
    g, u = np.asarray(fw["g"], np.float64), np.asarray(fw["u"], np.float64)
    R, hf = g.shape
    dst_row, offsets = fw["dst_row"], fw["offsets"]
    T, k = dst_row.shape
    h = w2.shape[2]
    g_err = np.zeros((R, hf)) if g_err is None else np.asarray(g_err, np.float64)
    u_err = np.zeros((R, hf)) if u_err is None else np.asarray(u_err, np.float64)
    out = dict(d_a=np.zeros((R, hf)), d_yp=np.zeros((R, h)), yp=np.zeros((R, h)))
    dev = np.zeros((R, h))
    ypo_abs = np.abs(np.asarray(fw["yp"], np.float64))
    for e in range(w1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ge, ue, dg, du = g[lo:hi], u[lo:hi], g_err[lo:hi], u_err[lo:hi]
        umax = np.abs(ue) + du
        silu_max = np.abs(silu(ge)) + 1.1 * dg
        a0 = silu(ge) * ue
        # fp32 evaluation of SiLU(G) U at the largest magnitudes, and the
        # rounding of A itself to fp32
        ev_a, _, _ = swiglu_eval_bound(np.abs(ge) + dg, umax, 0.0, silu_max, 0.0)
        d_eval = ev_a + F32_U * np.abs(a0)
        d_a = 1.1 * dg * umax + silu_max * du + d_eval
        out["d_a"][lo:hi] = d_eval
        qa, sp = rowq_spread_interval(a0, a0 - d_a, a0 + d_a)
        q2, s2 = quantize_cols(np.asarray(w2[e], np.float32))
        b2 = e4m3_decode(q2) * s2.astype(np.float64)[None, :]          # [hf, h]
        d_c = product_spread(qa, sp, b2.T, np.zeros_like(b2.T), hf)
        out["d_yp"][lo:hi] = fp32_sum_gamma(hf + 2) * ((np.abs(qa) + sp) @ np.abs(b2))
        # Yp is stored in fp32: the rescaled fp32 sum itself
        dev[lo:hi] = d_c
    out["yp"] = dev
    w = np.asarray(fw["w"], np.float64)
    w_err = np.zeros(w.shape) if w_err is None else np.asarray(w_err, np.float64)
    allow = np.zeros((T, h)); mag = np.zeros((T, h))
    for j in range(k):
        kept = dst_row[:, j] >= 0
        r = dst_row[kept, j]
        allow[kept] += np.abs(w[kept, j])[:, None] * dev[r] + w_err[kept, j][:, None] * (ypo_abs[r] + dev[r])
        mag[kept] += (np.abs(w[kept, j]) + w_err[kept, j])[:, None] * (ypo_abs[r] + dev[r])
    allow += fp32_sum_gamma(k) * mag
    out["y"] = allow * (1.0 + 2.0 ** -8)
    return out
