"""Algorithmic work of the MoE expert layer: FLOPs and HBM bytes per step.

Pure shape arithmetic, used for roofline fractions.  "Algorithmic" means
what the method must compute or move at least once: padding, re-reads and
scratch traffic are excluded.

Page formulas reproduced here (checked against the pages' printed values):
  * activation bytes ``b*s*h*2`` for BF16 and the dispatch bytes per token
    ``k*h*2`` -- research digest "MegaScale-MoE ... in Production", §3.2
    worked table;
  * per-GPU collective volumes of the attention / FFN layouts, Eqs. (1)-(4)
    of the same section (used only to size the multi-GPU design);
  * the compute/communication ratio ``R = 1.5 * h_ff * (B/P) * n/(n-1)``,
    same page §3.4.
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def expert_flops_fwd(R: int, h: int, h_ffn: int) -> int:
    """FC1 (two h x h_ffn products) + FC2 (one), 2 FLOPs per multiply-add."""
    return 6 * R * h * h_ffn


def expert_flops_bwd(R: int, h: int, h_ffn: int) -> int:
    """dA, dW2, dXp (two products), dW1, dW3: twice the forward."""
    return 12 * R * h * h_ffn


def router_flops(T: int, h: int, E: int) -> int:
    return 2 * T * h * E


def router_bytes(T, h, E, k, s_x):
    """Read x and W_g, write idx and w (4 B each)."""
    return T * h * s_x + h * E * s_x + T * k * 8


def permute_bytes(T, h, k, s_x, s_xp, scales=False):
    """Read each token row once, write k routed copies, read dst_row (4 B per
    row); FP8 adds a 4-byte scale per routed row."""
    R = T * k
    return T * h * s_x + R * h * s_xp + 4 * R + (4 * R if scales else 0)


def combine_bytes(T, h, k, s_yp, s_y):
    """Read the k routed rows of every token, write one row, read dst_row and w."""
    R = T * k
    return R * h * s_yp + T * h * s_y + 8 * R


def gemm_weight_bytes(E, h, h_ffn, s_w):
    return 3 * E * h * h_ffn * s_w


def activation_bytes(b, s, h, elem=2):
    return b * s * h * elem


def dispatch_bytes_per_token(k, h, elem=2):
    return k * h * elem


def tp_attn_volume(b, s, h, n, elem=2):
    """Eq. (1): tensor-parallel attention, per GPU per layer."""
    return 2 * b * s * h * elem * (n - 1) / n


def sp_attn_volume(b, s, h, n, m, elem=2):
    """Eq. (2): Ulysses sequence-parallel attention."""
    return tp_attn_volume(b, s, h, n, elem) * (2 + 2 / m) / n


def ep_ffn_volume(b, s, h, n, k, elem=2):
    """Eq. (3): expert-parallel all-to-all (dispatch + combine)."""
    return (k / n) * tp_attn_volume(b, s, h, n, elem)


def tp_ffn_volume(b, s, h, n, elem=2):
    """Eq. (4): tensor-parallel FFN."""
    return tp_attn_volume(b, s, h, n, elem)


def comp_comm_ratio(h_ff, bandwidth, peak, n):
    return 1.5 * h_ff * (bandwidth / peak) * n / (n - 1)


def workload_counts(wl) -> dict:
    """Every per-step figure for one workload (``moe_synth.Workload``)."""
    s_in = ELEM_BYTES[wl.storage]
    s_g = ELEM_BYTES[wl.dtype]
    R = wl.T * wl.k
    out = dict(
        R=R,
        flops_fwd=expert_flops_fwd(R, wl.h, wl.h_ffn),
        flops_fc1=4 * R * wl.h * wl.h_ffn,
        flops_fc2=2 * R * wl.h * wl.h_ffn,
        router_flops=router_flops(wl.T, wl.h, wl.E),
        router_bytes=router_bytes(wl.T, wl.h, wl.E, wl.k, s_in),
        permute_bytes=permute_bytes(wl.T, wl.h, wl.k, s_in, s_g, scales=wl.dtype == "fp8"),
        # the expert outputs Yp are kept in fp32 (4 bytes each)
        combine_bytes=combine_bytes(wl.T, wl.h, wl.k, 4, s_in),
        weight_bytes=gemm_weight_bytes(wl.E, wl.h, wl.h_ffn, s_g),
    )
    # bytes of every dispatch / combine launch of one step, in launch order
    out["permute_launches"] = [out["permute_bytes"]]
    out["combine_launches"] = [out["combine_bytes"]]
    if wl.backward:
        out["flops_bwd"] = expert_flops_bwd(R, wl.h, wl.h_ffn)
        # dY dispatched with the gate weights as row scales (4 B each read)
        dy_b = permute_bytes(wl.T, wl.h, wl.k, s_in, s_in) + 4 * R
        xg_b = permute_bytes(wl.T, wl.h, wl.k, s_in, s_in)      # x re-gathered
        if wl.dtype == "fp8":
            # dY only as per-token E4M3 codes with scale w * s per routed row:
            # the FP8 weight gradients gather w * dY and Xp from dY and x
            dyq_b = permute_bytes(wl.T, wl.h, wl.k, s_in, 1, scales=True) + 4 * R
            out["permute_launches"] += [dyq_b]
        else:
            out["permute_launches"] += [dy_b, xg_b]
        # dX of the expert path: no gate weights read, fp32 output (the router
        # backward adds its term and rounds once)
        out["combine_launches"].append(combine_bytes(wl.T, wl.h, wl.k, s_in, 4) - 4 * R)
        out["permute_bytes_bwd"] = sum(out["permute_launches"][1:])
        out["combine_bytes_bwd"] = out["combine_launches"][1]
    return out
