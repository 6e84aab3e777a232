"""Python binding of the C ABI, one function per entry point (same names).

Each function takes torch tensors (device memory) or ``None`` and forwards
their addresses, sizes and the current HIP stream to ``libmoe.so``.  No
arithmetic of the layer happens here.  ``MoELayer`` preallocates every buffer
of one layer call so a step launches kernels only.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MoeWeights, check, lib)

_TORCH_CODE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3,
               torch.uint8: MOE_FP8_E4M3}
_CODE_TORCH = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.uint8}


def dtype_code(t) -> int:
    return _TORCH_CODE[t if isinstance(t, torch.dtype) else t.dtype]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---- entry points ---------------------------------------------------------

def moe_packed_weight_bytes(which, E, h, h_ffn, dtype):
    return lib().moe_packed_weight_bytes(which, E, h, h_ffn, dtype)


def moe_pack_weights(w1, w3, w2, in_dtype, E, h, h_ffn, out_dtype, w13, w2_packed, w13_scale,
                     w2_scale, w13_bwd=None, w2_bwd=None, w13_bwd_scale=None, w2_bwd_scale=None,
                     stream=None):
    return check(lib().moe_pack_weights(_p(w1), _p(w3), _p(w2), in_dtype, E, h, h_ffn, out_dtype,
                                        _p(w13), _p(w2_packed), _p(w13_scale), _p(w2_scale),
                                        _p(w13_bwd), _p(w2_bwd), _p(w13_bwd_scale), _p(w2_bwd_scale),
                                        _s(stream)))


def moe_route(x, w_gate, bias, logits, T, h, E, k, dtype, topk_idx, topk_w, stream=None):
    return check(lib().moe_route(_p(x), _p(w_gate), _p(bias), _p(logits), T, h, E, k, dtype,
                                 _p(topk_idx), _p(topk_w), _s(stream)))


def moe_permute_workspace_size(T, E, k):
    return lib().moe_permute_workspace_size(T, E, k)


def moe_permute(src, src_dtype, topk_idx, row_scale, T, h, E, k, counts, offsets, dst_row, src_tok,
                dst, dst_dtype, dst_scale, ws, ws_bytes, stream=None):
    return check(lib().moe_permute(_p(src), src_dtype, _p(topk_idx), _p(row_scale), T, h, E, k,
                                   _p(counts), _p(offsets), _p(dst_row), _p(src_tok), _p(dst),
                                   dst_dtype, _p(dst_scale), _p(ws), ws_bytes, _s(stream)))


def moe_permute_noalloc(src, src_dtype, topk_idx, row_scale, T, h, E, k, counts, offsets, dst_row,
                        src_tok, dst, dst_dtype, dst_scale, stream=None):
    return check(lib().moe_permute_noalloc(_p(src), src_dtype, _p(topk_idx), _p(row_scale), T, h, E, k,
                                           _p(counts), _p(offsets), _p(dst_row), _p(src_tok), _p(dst),
                                           dst_dtype, _p(dst_scale), _s(stream)))


def moe_permute_local_workspace_size(T, e_count, k):
    return lib().moe_permute_local_workspace_size(T, e_count, k)


def moe_permute_local(src, src_dtype, topk_idx, row_scale, T, h, E, k, e_lo, e_count, counts, offsets,
                      dst_row, src_tok, dst, dst_dtype, dst_scale, ws, ws_bytes, stream=None):
    return check(lib().moe_permute_local(_p(src), src_dtype, _p(topk_idx), _p(row_scale), T, h, E, k,
                                         e_lo, e_count, _p(counts), _p(offsets), _p(dst_row),
                                         _p(src_tok), _p(dst), dst_dtype, _p(dst_scale), _p(ws),
                                         ws_bytes, _s(stream)))


def moe_capacity_drop_workspace_size(T, E, k):
    return lib().moe_capacity_drop_workspace_size(T, E, k)


def moe_capacity_drop(topk_idx, logits, T, E, k, group, capacity, topk_idx_out, ws, ws_bytes,
                      stream=None):
    return check(lib().moe_capacity_drop(_p(topk_idx), _p(logits), T, E, k, group, capacity,
                                         _p(topk_idx_out), _p(ws), ws_bytes, _s(stream)))


def moe_grouped_workspace_size(rows, h, h_ffn, E, dtype):
    return lib().moe_grouped_workspace_size(rows, h, h_ffn, E, dtype)


def moe_grouped_swiglu_fwd(xp, xp_scale, W, offsets, rows, h13_save, yp, yp_dtype, ws, ws_bytes,
                           stream=None):
    return check(lib().moe_grouped_swiglu_fwd(_p(xp), _p(xp_scale), ctypes.byref(W), _p(offsets),
                                              rows, _p(h13_save), _p(yp), yp_dtype, _p(ws), ws_bytes,
                                              _s(stream)))


def moe_grouped_bwd_workspace_size(rows, h, h_ffn, E, dtype):
    return lib().moe_grouped_bwd_workspace_size(rows, h, h_ffn, E, dtype)


def moe_grouped_swiglu_bwd(dyp, xp, h13_save, W, offsets, rows, dxp, dw1, dw3, dw2, ws, ws_bytes,
                           stream=None):
    return check(lib().moe_grouped_swiglu_bwd(_p(dyp), _p(xp), _p(h13_save), ctypes.byref(W),
                                              _p(offsets), rows, _p(dxp), _p(dw1), _p(dw3),
                                              _p(dw2), _p(ws), ws_bytes, _s(stream)))


def moe_combine(yp, yp_dtype, dst_row, topk_w, T, h, k, y, y_dtype, stream=None):
    return check(lib().moe_combine(_p(yp), yp_dtype, _p(dst_row), _p(topk_w), T, h, k, _p(y),
                                   y_dtype, _s(stream)))


def moe_router_bwd_workspace_size(T, h, E):
    return lib().moe_router_bwd_workspace_size(T, h, E)


def moe_router_bwd(dy, yp, yp_dtype, dst_row, topk_idx, topk_w, logits, counts, T, h, E, k, alpha,
                   dtype, x, w_gate, dx_in, dx, dlogits, dw_gate, dbias, ws, ws_bytes, stream=None):
    return check(lib().moe_router_bwd(_p(dy), _p(yp), yp_dtype, _p(dst_row), _p(topk_idx), _p(topk_w),
                                      _p(logits), _p(counts), T, h, E, k, float(alpha), dtype, _p(x),
                                      _p(w_gate), _p(dx_in), _p(dx), _p(dlogits), _p(dw_gate),
                                      _p(dbias), _p(ws), ws_bytes, _s(stream)))


def moe_router_aux_workspace_size(T, E):
    return lib().moe_router_aux_workspace_size(T, E)


def moe_router_aux_loss(logits, counts, T, E, k, alpha, loss, ws, ws_bytes, stream=None):
    return check(lib().moe_router_aux_loss(_p(logits), _p(counts), T, E, k, float(alpha), _p(loss),
                                           _p(ws), ws_bytes, _s(stream)))


def moe_grouped_bwd_fp8_workspace_size(rows, h, h_ffn, E):
    return lib().moe_grouped_bwd_fp8_workspace_size(rows, h, h_ffn, E)


def moe_grouped_swiglu_bwd_fp8(dyp_q, dyp_scale, dyp, xp, h13_save, W, offsets, rows, dxp, dw1, dw3,
                               dw2, ws, ws_bytes, stream=None):
    return check(lib().moe_grouped_swiglu_bwd_fp8(_p(dyp_q), _p(dyp_scale), _p(dyp), _p(xp),
                                                  _p(h13_save), ctypes.byref(W), _p(offsets), rows,
                                                  _p(dxp), _p(dw1), _p(dw3), _p(dw2), _p(ws), ws_bytes,
                                                  _s(stream)))


def moe_grouped_swiglu_bwd_fp8_tok(dyp_q, dyp_scale, dy, x, dst_row, topk_w, T, k, h13_save, W, offsets, rows,
                                   dxp, dw1, dw3, dw2, ws, ws_bytes, stream=None):
    return check(lib().moe_grouped_swiglu_bwd_fp8_tok(_p(dyp_q), _p(dyp_scale), _p(dy), _p(x), _p(dst_row),
                                                      _p(topk_w), T, k, _p(h13_save), ctypes.byref(W),
                                                      _p(offsets), rows, _p(dxp), _p(dw1), _p(dw3), _p(dw2),
                                                      _p(ws), ws_bytes, _s(stream)))


def moe_dispatch_swiglu_fwd_workspace_size(T, k, h, h_ffn, E):
    return lib().moe_dispatch_swiglu_fwd_workspace_size(T, k, h, h_ffn, E)


def moe_dispatch_swiglu_fwd(x, topk_idx, T, k, counts, offsets, dst_row, src_tok, W, xp, h13_save, yp, yp_dtype,
                            status, ws, ws_bytes, stream=None):
    return check(lib().moe_dispatch_swiglu_fwd(_p(x), _p(topk_idx), T, k, _p(counts), _p(offsets), _p(dst_row),
                                               _p(src_tok), ctypes.byref(W), _p(xp), _p(h13_save), _p(yp), yp_dtype,
                                               _p(status), _p(ws), ws_bytes, _s(stream)))


def moe_dispatch_swiglu_fwd_wait_selftest(x, topk_idx, T, k, counts, offsets, dst_row, src_tok, W, xp, h13_save,
                                          yp, yp_dtype, status, ws, ws_bytes, stream=None):
    return check(lib().moe_dispatch_swiglu_fwd_wait_selftest(
        _p(x), _p(topk_idx), T, k, _p(counts), _p(offsets), _p(dst_row), _p(src_tok), ctypes.byref(W), _p(xp),
        _p(h13_save), _p(yp), yp_dtype, _p(status), _p(ws), ws_bytes, _s(stream)))


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> int:
    return lib().moe_version()


def moe_fp8_convert_selftest(mismatches, stream=None):
    return check(lib().moe_fp8_convert_selftest(_p(mismatches), _s(stream)))


# ---- one preallocated layer ------------------------------------------------

class PackedWeights:
    """Expert weights packed (and for FP8 quantized) by ``moe_pack_weights``."""

    def __init__(self, w1, w3, w2, out_dtype: int, backward: bool = False, stream=None):
        E, h, hf = w1.shape
        dev = w1.device
        in_dt = dtype_code(w1)
        self.dtype, self.E, self.h, self.h_ffn = out_dtype, E, h, hf
        sz = lambda which: moe_packed_weight_bytes(which, E, h, hf, out_dtype)
        self.w13 = torch.empty(sz(0), dtype=torch.uint8, device=dev)
        self.w2 = torch.empty(sz(1), dtype=torch.uint8, device=dev)
        fp8 = out_dtype == MOE_FP8_E4M3
        self.w13_scale = torch.empty(E, 2 * hf, dtype=torch.float32, device=dev) if fp8 else None
        self.w2_scale = torch.empty(E, h, dtype=torch.float32, device=dev) if fp8 else None
        self.w13_bwd = torch.empty(sz(4), dtype=torch.uint8, device=dev) if backward else None
        self.w2_bwd = torch.empty(sz(5), dtype=torch.uint8, device=dev) if backward else None
        bq = backward and fp8
        self.w13_bwd_scale = torch.empty(E, h, dtype=torch.float32, device=dev) if bq else None
        self.w2_bwd_scale = torch.empty(E, hf, dtype=torch.float32, device=dev) if bq else None
        moe_pack_weights(w1, w3, w2, in_dt, E, h, hf, out_dtype, self.w13, self.w2,
                         self.w13_scale, self.w2_scale, self.w13_bwd, self.w2_bwd,
                         self.w13_bwd_scale, self.w2_bwd_scale, stream)
        ptr = lambda t: None if t is None else t.data_ptr()
        self.struct = MoeWeights(out_dtype, E, h, hf, self.w13.data_ptr(), self.w2.data_ptr(),
                                 ptr(self.w13_scale), ptr(self.w2_scale), ptr(self.w13_bwd),
                                 ptr(self.w2_bwd), ptr(self.w13_bwd_scale), ptr(self.w2_bwd_scale))


class MoELayer:
    """Buffers and launch sequence of one MoE layer call on a fixed shape.

    forward(): route -> permute (index + copy) -> grouped SwiGLU -> combine.
    backward(): weighted dispatch of dY -> grouped backward -> combine (dX).
    The expert outputs Yp are kept in fp32 (``yp_dtype``; MOE_BF16 stores
    them rounded, half the bytes).
    """

    def __init__(self, T, h, h_ffn, E, k, dtype: int, device="cuda", save_for_backward=False,
                 yp_dtype: int = MOE_F32):
        self.T, self.h, self.h_ffn, self.E, self.k, self.dtype = T, h, h_ffn, E, k, dtype
        R = T * k
        self.R = R
        dev = torch.device(device)
        io = torch.float32 if dtype == MOE_F32 else torch.bfloat16
        self.io_code = MOE_F32 if dtype == MOE_F32 else MOE_BF16
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.logits = torch.empty(T, E, **f32)
        self.topk_idx = torch.empty(T, k, **i32)
        self.topk_w = torch.empty(T, k, **f32)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.dst_row = torch.empty(T, k, **i32)
        self.src_tok = torch.empty(R, **i32)
        self.pws_bytes = moe_permute_workspace_size(T, E, k)
        self.pws = torch.empty(max(self.pws_bytes, 256), dtype=torch.uint8, device=dev)
        xp_dt = torch.uint8 if dtype == MOE_FP8_E4M3 else io
        self.xp = torch.empty(R, h, dtype=xp_dt, device=dev)
        self.xp_scale = torch.empty(R, **f32) if dtype == MOE_FP8_E4M3 else None
        self.h13 = torch.empty(R, 2 * h_ffn, dtype=torch.bfloat16, device=dev) if save_for_backward else None
        self.yp_code = MOE_F32 if dtype == MOE_F32 else yp_dtype
        self.yp = torch.empty(R, h, dtype=torch.float32 if self.yp_code == MOE_F32 else torch.bfloat16,
                              device=dev)
        self.y = torch.empty(T, h, dtype=io, device=dev)
        self.gws_bytes = moe_grouped_workspace_size(R, h, h_ffn, E, dtype)
        self.gws = torch.empty(max(self.gws_bytes, 256), dtype=torch.uint8, device=dev)
        self.bwd_ready = False

    def forward(self, x, w_gate, bias, W: PackedWeights, logits_in=None, capacity=None, group=1,
                stream=None, arrival=False):
        """One layer forward.  With ``capacity``, pairs beyond the capacity of
        each group of ``group`` experts are dropped by affinity before the
        dispatch (moe_capacity_drop).  With ``arrival`` (BF16), the dispatch
        copy and FC1 overlap by tile arrival (moe_dispatch_swiglu_fwd; the
        status word is ``self.arrival_status``)."""
        T, h, E, k = self.T, self.h, self.E, self.k
        if logits_in is None:
            moe_route(x, w_gate, bias, self.logits, T, h, E, k, dtype_code(x), self.topk_idx,
                      self.topk_w, stream)
            self.logits_used = self.logits
        else:
            moe_route(None, None, None, logits_in, T, h, E, k, dtype_code(logits_in),
                      self.topk_idx, self.topk_w, stream)
            self.logits_used = logits_in
        if capacity is not None:
            if not hasattr(self, "cws"):
                self.cws_bytes = moe_capacity_drop_workspace_size(T, E, k)
                self.cws = torch.empty(max(self.cws_bytes, 256), dtype=torch.uint8, device=self.y.device)
            moe_capacity_drop(self.topk_idx, self.logits_used, T, E, k, group, capacity, self.topk_idx,
                              self.cws, self.cws_bytes, stream)
        if arrival:
            if not hasattr(self, "aws"):
                self.aws_bytes = moe_dispatch_swiglu_fwd_workspace_size(T, k, h, self.h_ffn, E)
                self.aws = torch.empty(max(self.aws_bytes, 256), dtype=torch.uint8, device=self.y.device)
                self.arrival_status = torch.zeros(1, dtype=torch.int32, device=self.y.device)
            moe_dispatch_swiglu_fwd(x, self.topk_idx, T, k, self.counts, self.offsets, self.dst_row, self.src_tok,
                                    W.struct, self.xp, self.h13, self.yp, self.yp_code, self.arrival_status,
                                    self.aws, self.aws_bytes, stream)
        else:
            moe_permute(x, dtype_code(x), self.topk_idx, None, T, h, E, k, self.counts, self.offsets,
                        self.dst_row, self.src_tok, self.xp, self.dtype, self.xp_scale, self.pws,
                        self.pws_bytes, stream)
            moe_grouped_swiglu_fwd(self.xp, self.xp_scale, W.struct, self.offsets, self.R, self.h13,
                                   self.yp, self.yp_code, self.gws, self.gws_bytes, stream)
        moe_combine(self.yp, self.yp_code, self.dst_row, self.topk_w, T, h, k, self.y,
                    self.io_code, stream)
        return self.y

    def _alloc_bwd(self):
        dev = self.y.device
        R, h, hf, E = self.R, self.h, self.h_ffn, self.E
        self.dxp = torch.empty(R, h, dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty(self.T, h, dtype=torch.bfloat16, device=dev)
        self.dw1 = torch.empty(E, h, hf, dtype=torch.float32, device=dev)
        self.dw3 = torch.empty(E, h, hf, dtype=torch.float32, device=dev)
        self.dw2 = torch.empty(E, hf, h, dtype=torch.float32, device=dev)
        if self.dtype == MOE_FP8_E4M3:
            self.dyp_q = torch.empty(R, h, dtype=torch.uint8, device=dev)
            self.dyp_s = torch.empty(R, dtype=torch.float32, device=dev)
            self.bws_bytes = moe_grouped_bwd_fp8_workspace_size(R, h, hf, E)
        else:
            self.dyp = torch.empty(R, h, dtype=torch.bfloat16, device=dev)
            self.bws_bytes = moe_grouped_bwd_workspace_size(R, h, hf, E, self.dtype)
        self.bws = torch.empty(max(self.bws_bytes, 256), dtype=torch.uint8, device=dev)
        self.bwd_ready = True

    def aux_loss(self, alpha, stream=None):
        """Load-balance loss of the last forward's routing (a device scalar)."""
        if not hasattr(self, "aux_ws"):
            self.aux_ws_bytes = moe_router_aux_workspace_size(self.T, self.E)
            self.aux_ws = torch.empty(max(self.aux_ws_bytes, 256), dtype=torch.uint8, device=self.y.device)
            self.aux = torch.empty(4, dtype=torch.float32, device=self.y.device)
        moe_router_aux_loss(self.logits_used, self.counts, self.T, self.E, self.k, alpha, self.aux,
                            self.aux_ws, self.aux_ws_bytes, stream)
        return self.aux[0]

    def _alloc_router_bwd(self):
        dev, T, h, E = self.y.device, self.T, self.h, self.E
        f32 = dict(dtype=torch.float32, device=dev)
        self.dx_expert = torch.empty(T, h, **f32)
        self.dlogits = torch.empty(T, E, **f32)
        self.dw_gate = torch.empty(h, E, **f32)
        self.dbias = torch.empty(E, **f32)
        self.rws_bytes = moe_router_bwd_workspace_size(T, h, E)
        self.rws = torch.empty(max(self.rws_bytes, 256), dtype=torch.uint8, device=dev)

    def backward(self, dy, x, W: PackedWeights, w_gate=None, alpha=0.0, stream=None):
        """dX (expert path, plus the router path when ``w_gate`` is given),
        per-expert dW1/dW3/dW2 and, with ``w_gate``, dW_g / d(bias) / dL
        including the balance loss of weight ``alpha``."""
        if not self.bwd_ready:
            self._alloc_bwd()
        T, h, E, k = self.T, self.h, self.E, self.k
        if self.dtype == MOE_FP8_E4M3:
            # dY codes per token, routed row scale w * s; the weight gradients'
            # operands w * dY and Xp are gathered from dY and x where they are
            # quantized (no routed bf16 copies)
            moe_permute(dy, MOE_BF16, None, self.topk_w, T, h, E, k, None, None, self.dst_row, None,
                        self.dyp_q, MOE_FP8_E4M3, self.dyp_s, None, 0, stream)
            moe_grouped_swiglu_bwd_fp8_tok(self.dyp_q, self.dyp_s, dy, x, self.dst_row, self.topk_w, T, k,
                                           self.h13, W.struct, self.offsets, self.R, self.dxp, self.dw1,
                                           self.dw3, self.dw2, self.bws, self.bws_bytes, stream)
        else:
            # dYp = w * dY in dispatch order; Xp re-gathered from x (index reused)
            moe_permute(dy, MOE_BF16, None, self.topk_w, T, h, E, k, None, None, self.dst_row, None,
                        self.dyp, MOE_BF16, None, None, 0, stream)
            moe_permute(x, MOE_BF16, None, None, T, h, E, k, None, None, self.dst_row, None,
                        self.xp, MOE_BF16, None, None, 0, stream)
            moe_grouped_swiglu_bwd(self.dyp, self.xp, self.h13, W.struct, self.offsets, self.R,
                                   self.dxp, self.dw1, self.dw3, self.dw2, self.bws, self.bws_bytes,
                                   stream)
        if w_gate is None:
            moe_combine(self.dxp, MOE_BF16, self.dst_row, None, T, h, k, self.dx, MOE_BF16, stream)
            return self.dx
        if not hasattr(self, "dw_gate"):
            self._alloc_router_bwd()
        # expert path in fp32, then the router path adds dL W_g^T and rounds once
        moe_combine(self.dxp, MOE_BF16, self.dst_row, None, T, h, k, self.dx_expert, MOE_F32, stream)
        moe_router_bwd(dy, self.yp, self.yp_code, self.dst_row, self.topk_idx, self.topk_w, self.logits_used,
                       self.counts, T, h, E, k, alpha, dtype_code(dy), x, w_gate, self.dx_expert,
                       self.dx, self.dlogits, self.dw_gate, self.dbias, self.rws, self.rws_bytes,
                       stream)
        return self.dx


def moe_timing_enable(on: bool) -> int:
    return check(lib().moe_timing_enable(1 if on else 0))


def moe_timing_report() -> dict:
    """{kernel: (launches, total_ms)} recorded since timing was enabled."""
    buf = ctypes.create_string_buffer(4096)
    check(lib().moe_timing_report(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out
