"""Sub-problems of the FP8 backward that the oracle can finish at full size.

The FP8 backward quantizes dY per token, dG|dU and A per routed row for the
activation-gradient products, and the weight-gradient operands per channel
over one expert's rows (the weights per channel of each product, per expert).
So the weight gradients of one expert depend on that expert's routed rows
only, and the dX row of a token on its own routed rows only.  A sub-problem
hands the oracle those rows, each as a token of its own (k = 1), with the
expert weights of the experts involved; `tests/test_oracle_fp8.py` checks that
the oracle's results on such sub-problems equal its whole-layer results.

Test infrastructure: plain NumPy on the oracle's argument layout.
"""
import numpy as np


def gu_src_columns(hf):
    """Source column (in [G | U]) of each column of the kept [rows][2hf]
    array, whose 32-column groups of G and U alternate."""
    p = np.arange(2 * hf)
    return np.where((p // 32) % 2 == 1, hf, 0) + (p // 64) * 32 + p % 32


def unpack_gu(packed):
    """G and U ([rows][hf] each) from the kept interleaved [rows][2hf] array."""
    hf = packed.shape[1] // 2
    cat = np.empty_like(packed)
    cat[:, gu_src_columns(hf)] = packed
    return cat[:, :hf], cat[:, hf:]


def subproblem(dy, x, w, idx, dst_row, g_rows, u_rows, w1, w3, w2, toks, slots, experts):
    """`layer_backward_fp8` arguments for the routed rows (toks[i], slots[i]),
    which must come grouped by expert in the order of `experts`.  ``w`` [T, k]
    gate weights; ``g_rows`` / ``u_rows`` the kept G / U of every routed row
    (indexed by dst_row); w1, w3, w2 all experts' weights (fp32 arrays)."""
    toks, slots = np.asarray(toks), np.asarray(slots)
    ex = idx[toks, slots]
    offs = np.concatenate([[0], np.cumsum([np.count_nonzero(ex == e) for e in experts])]).astype(np.int64)
    assert offs[-1] == len(toks)
    assert all((ex[offs[i]:offs[i + 1]] == e).all() for i, e in enumerate(experts)), "rows not grouped"
    rows = dst_row[toks, slots]
    experts = list(experts)
    return (dy[toks], x[toks], np.asarray(w, np.float64)[toks, slots][:, None], np.arange(len(toks))[:, None],
            offs, w1[experts], w3[experts], w2[experts], g_rows[rows], u_rows[rows])


def expert_rows(e, offsets, dst_row, src_tok):
    """(toks, slots) of expert e's routed rows, in row order."""
    rows = np.arange(offsets[e], offsets[e + 1])
    toks = src_tok[rows]
    slots = np.array([np.nonzero(dst_row[t] == r)[0][0] for t, r in zip(toks, rows)], dtype=np.int64)
    return toks, slots


def token_rows(tok_s, idx):
    """(toks, slots, experts) of every routed row of the tokens tok_s, grouped
    by expert."""
    pairs = sorted((int(idx[t, j]), int(t), j) for t in tok_s for j in range(idx.shape[1]))
    toks = np.array([p[1] for p in pairs]); slots = np.array([p[2] for p in pairs])
    return toks, slots, sorted(set(p[0] for p in pairs))


def token_sum(v, tok_s, toks):
    """Per-token sums of per-row values v (rows belonging to toks)."""
    out = np.zeros((len(tok_s),) + v.shape[1:])
    np.add.at(out, np.searchsorted(tok_s, toks), v)
    return out
