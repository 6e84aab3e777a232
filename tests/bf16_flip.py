"""Per-element allowance for one BF16 operand rounded the other way.

A BF16 training step rounds its matrix-product operands (dYp, the kept G and
U, A, dG, dU) to BF16 from fp32 values; the oracle with BF16 operands rounds
the same quantities from fp64 values.  Where the fp32 and fp64 values of one
operand lie on either side of a BF16 rounding boundary, the two round to
neighbouring BF16 values, and every weight-gradient element that sums a term
with that operand moves by that term's change.  An indexing or accumulation
error moves whole terms instead; the allowance is one BF16 step of one term.

For each weight-gradient element, the allowance is the largest change that a
single such flip can make to it, over the terms of its sum:
  dW1[i, n] = sum_r Xp[r, i] dG[r, n]   flips of dG[r, n], or of G[r, n] or
                                        U[r, n], which form dG[r, n]
  dW3[i, n] = sum_r Xp[r, i] dU[r, n]   flips of dU[r, n] or of G[r, n]
  dW2[n, m] = sum_r A[r, n] dYp[r, m]   flips of A[r, n] (or G, U) or dYp[r, m]
A flip of G or U is evaluated through the elementwise SwiGLU formulas at the
neighbouring BF16 value, plus one step of the re-rounded result.  Flips of
dYp inside dA = dYp W2^T (one term of a sum over h) are not counted.

Test infrastructure: written with the oracle's own functions and fp64 NumPy.
"""
import numpy as np

from oracle import moe_ref as ref


def bf16_step(v):
    """Spacing of BF16 values just above |v| (8 significant bits); 0 for 0."""
    v = np.asarray(v, np.float64)
    _, ex = np.frexp(v)
    return np.where(v != 0, np.ldexp(1.0, ex - 8), 0.0)


def _max_outer(p, q, chunk=32):
    """out[a, b] = max_r p[r, a] * q[r, b] for non-negative p, q."""
    out = np.zeros((p.shape[1], q.shape[1]))
    for r0 in range(0, p.shape[0], chunk):
        blk = p[r0:r0 + chunk, :, None] * q[r0:r0 + chunk, None, :]
        np.maximum(out, blk.max(axis=0), out=out)
    return out


def _dg(da, g, u):
    s = ref.sigmoid(g)
    return da * u * s * (1.0 + g * (1.0 - s))


def _du(da, g):
    return da * ref.silu(g)


def _a(g, u):
    return ref.silu(g) * u


def _flip_g(f, g):
    """Largest |f(g +- one step) - f(g)| elementwise."""
    st = bf16_step(g)
    f0 = f(g)
    return np.maximum(np.abs(f(g + st) - f0), np.abs(f(g - st) - f0))


def weight_grad_flip_allowance(dy, x, w, dst_row, offsets, w1, w3, w2):
    """Allowance per element of dW1, dW3 and dW2 (shapes of w1, w3, w2).

    Arguments as for the oracle's ``layer_backward``; the operands are
    rebuilt as its BF16-operand mode rounds them.
    """
    rb = ref.round_bf16
    xp = ref.permute(np.asarray(x, np.float64), dst_row)
    dyp = rb(ref.permute(np.asarray(dy, np.float64), dst_row, row_scale=w))
    out = {"dw1": np.zeros(w1.shape), "dw3": np.zeros(w3.shape), "dw2": np.zeros(w2.shape)}
    for e in range(w1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W1 = np.asarray(w1[e], np.float64); W3 = np.asarray(w3[e], np.float64)
        W2 = np.asarray(w2[e], np.float64)
        xe, dye = xp[lo:hi], dyp[lo:hi]
        g, u = rb(xe @ W1), rb(xe @ W3)
        da = dye @ W2.T
        dg, du, a = rb(_dg(da, g, u)), rb(_du(da, g)), rb(_a(g, u))
        su = bf16_step(u)
        d_dg = bf16_step(dg) + np.maximum(_flip_g(lambda gg: _dg(da, gg, u), g),
                                          np.abs(_dg(da, g, u + su) - _dg(da, g, u)))
        d_du = bf16_step(du) + _flip_g(lambda gg: _du(da, gg), g)
        d_a = bf16_step(a) + np.maximum(_flip_g(lambda gg: _a(gg, u), g), np.abs(_a(g, u + su) - _a(g, u)))
        ax = np.abs(xe)
        out["dw1"][e] = _max_outer(ax, d_dg)
        out["dw3"][e] = _max_outer(ax, d_du)
        out["dw2"][e] = np.maximum(_max_outer(d_a, np.abs(dye)), _max_outer(np.abs(a), bf16_step(dye)))
    return out
