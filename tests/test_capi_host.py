"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, and rejects bad arguments before any HIP
call (so the error paths run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_24_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libmoe.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "moe_route" in names and "moe_grouped_swiglu_fwd" in names and len(names) >= 12
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(L.SIGNATURES)
    assert lib.moe_version() == 4


A = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first
U = ctypes.c_void_p((1 << 20) + 4)  # misaligned


def test_route_validation():
    lib = L.lib()
    ok_args = dict(x=A, wg=A, bias=None, logits=None, T=16, h=64, E=8, k=2, dt=L.MOE_BF16, idx=A, w=A)

    def call(**kw):
        a = {**ok_args, **kw}
        return lib.moe_route(a["x"], a["wg"], a["bias"], a["logits"], a["T"], a["h"], a["E"], a["k"],
                             a["dt"], a["idx"], a["w"], None)
    assert call(T=-1) == L.MOE_ERR_ARG
    assert call(k=9) == L.MOE_ERR_ARG
    assert call(k=0) == L.MOE_ERR_ARG
    assert call(E=0) == L.MOE_ERR_SHAPE
    assert call(E=L.MOE_MAX_EXPERTS + 1) == L.MOE_ERR_SHAPE
    assert call(idx=None) == L.MOE_ERR_ARG
    assert call(idx=U) == L.MOE_ERR_ARG
    assert call(dt=L.MOE_FP8_E4M3) == L.MOE_ERR_DTYPE
    assert call(h=96) == L.MOE_ERR_SHAPE
    assert call(x=None) == L.MOE_ERR_ARG        # logits-in mode needs logits
    assert b"logits" in lib.moe_last_error()
    assert call(T=0) == L.MOE_OK                # empty batch: nothing to launch


def test_permute_validation():
    lib = L.lib()
    need = lib.moe_permute_workspace_size(1000, 8, 2)
    assert need >= 4 * 8

    def call(src=A, sdt=L.MOE_BF16, idx=A, T=1000, h=64, E=8, k=2, dst=A, ddt=L.MOE_BF16, scale=None,
             ws=A, wsb=None, row_scale=None):
        return lib.moe_permute(src, sdt, idx, row_scale, T, h, E, k, A, A, A, A, dst, ddt, scale, ws,
                               need if wsb is None else wsb, None)
    assert call(h=12) == L.MOE_ERR_SHAPE
    assert call(sdt=L.MOE_F32) == L.MOE_ERR_DTYPE
    assert call(ddt=L.MOE_FP8_E4M3) == L.MOE_ERR_ARG            # fp8 needs scales
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(ws=None) == L.MOE_ERR_WORKSPACE
    assert call(dst=None) == L.MOE_ERR_ARG
    assert call(k=3, E=2) == L.MOE_ERR_ARG


def test_grouped_validation():
    lib = L.lib()
    W = L.MoeWeights(L.MOE_BF16, 8, 256, 384, A.value, A.value, None, None)
    need = lib.moe_grouped_workspace_size(512, 256, 384, 8, L.MOE_BF16)
    assert need >= 512 * 384 * 2

    def call(W=W, rows=512, ws=A, wsb=need, save=None, scale=None, ypdt=L.MOE_F32):
        return lib.moe_grouped_swiglu_fwd(A, scale, ctypes.byref(W), A, rows, save, A, ypdt, ws, wsb, None)
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(rows=-1) == L.MOE_ERR_ARG
    assert call(rows=0) == L.MOE_OK
    bad = L.MoeWeights(L.MOE_BF16, 8, 200, 384, A.value, A.value, None, None)
    assert call(W=bad) == L.MOE_ERR_SHAPE
    bad = L.MoeWeights(7, 8, 256, 384, A.value, A.value, None, None)
    assert call(W=bad) == L.MOE_ERR_DTYPE
    assert call(ypdt=L.MOE_FP8_E4M3) == L.MOE_ERR_DTYPE
    f32w = L.MoeWeights(L.MOE_F32, 8, 256, 384, A.value, A.value, None, None)
    assert call(W=f32w, ypdt=L.MOE_BF16) == L.MOE_ERR_DTYPE   # fp32 weights keep fp32 outputs
    f8 = L.MoeWeights(L.MOE_FP8_E4M3, 8, 256, 384, A.value, A.value, None, None)
    assert call(W=f8) == L.MOE_ERR_ARG                    # fp8 weights need scales
    f32 = L.MoeWeights(L.MOE_F32, 8, 256, 384, A.value, A.value, None, None)
    assert call(W=f32, save=A) == L.MOE_ERR_DTYPE         # G|U kept only for bf16
    assert lib.moe_grouped_swiglu_bwd(A, A, A, ctypes.byref(f32), A, 512, A, A, A, A, A, 1 << 30,
                                      None) == L.MOE_ERR_DTYPE
    # bf16 weights without the backward layouts
    assert lib.moe_grouped_swiglu_bwd(A, A, A, ctypes.byref(W), A, 512, A, A, A, A, A, 1 << 30,
                                      None) == L.MOE_ERR_ARG
    Wb = L.MoeWeights(L.MOE_BF16, 8, 256, 384, A.value, A.value, None, None, A.value, A.value, None, None)
    need = lib.moe_grouped_bwd_workspace_size(512, 256, 384, 8, L.MOE_BF16)
    assert need > 0
    assert lib.moe_grouped_swiglu_bwd(A, A, A, ctypes.byref(Wb), A, 512, A, A, A, A, A, need - 1,
                                      None) == L.MOE_ERR_WORKSPACE


def test_combine_and_pack_validation():
    lib = L.lib()
    assert lib.moe_combine(A, L.MOE_BF16, A, A, 10, 12, 2, A, L.MOE_BF16, None) == L.MOE_ERR_SHAPE
    assert lib.moe_combine(A, L.MOE_FP8_E4M3, A, A, 10, 16, 2, A, L.MOE_BF16, None) == L.MOE_ERR_DTYPE
    assert lib.moe_combine(A, L.MOE_BF16, A, None, 0, 16, 2, A, L.MOE_BF16, None) == L.MOE_OK
    assert lib.moe_pack_weights(A, A, A, L.MOE_F32, 8, 256, 384, L.MOE_BF16, A, A, None, None,
                                None, None, None, None, None) == L.MOE_ERR_DTYPE
    assert lib.moe_pack_weights(A, A, A, L.MOE_BF16, 8, 256, 384, L.MOE_FP8_E4M3, A, A, None, None,
                                None, None, None, None, None) == L.MOE_ERR_ARG
    assert lib.moe_pack_weights(A, A, A, L.MOE_BF16, 8, 256, 384, L.MOE_FP8_E4M3, A, A, A, A,
                                A, A, None, A, None) == L.MOE_ERR_ARG   # FP8 w13_bwd needs its scales
    assert lib.moe_pack_weights(A, A, A, L.MOE_F32, 8, 256, 384, L.MOE_F32, A, A, None, None,
                                A, A, None, None, None) == L.MOE_ERR_DTYPE   # no fp32 backward layouts
    assert lib.moe_packed_weight_bytes(4, 8, 256, 384, L.MOE_BF16) == 8 * 256 * 768 * 2
    assert lib.moe_packed_weight_bytes(5, 8, 256, 384, L.MOE_FP8_E4M3) == 8 * 384 * 256
    assert lib.moe_packed_weight_bytes(6, 8, 256, 384, L.MOE_FP8_E4M3) == 8 * 256 * 4
    assert lib.moe_packed_weight_bytes(7, 8, 256, 384, L.MOE_BF16) == 0
    assert lib.moe_packed_weight_bytes(0, 8, 256, 384, L.MOE_BF16) == 8 * 768 * 256 * 2
    assert lib.moe_packed_weight_bytes(3, 8, 256, 384, L.MOE_FP8_E4M3) == 8 * 256 * 4


def test_router_bwd_validation():
    lib = L.lib()
    T, h, E, k = 100, 128, 8, 2
    need = lib.moe_router_bwd_workspace_size(T, h, E)
    assert need > 0 and lib.moe_router_bwd_workspace_size(0, h, E) == 0
    ok = dict(dy=A, yp=A, ypdt=L.MOE_F32, dst=A, idx=A, w=A, lg=A, cnt=A, T=T, h=h, E=E, k=k, alpha=0.01,
              dt=L.MOE_BF16, x=A, wg=A, dxin=None, dx=ctypes.c_void_p(2 << 20), dl=None, dwg=A, db=None,
              ws=A, wsb=need)

    def call(**kw):
        a = {**ok, **kw}
        return lib.moe_router_bwd(a["dy"], a["yp"], a["ypdt"], a["dst"], a["idx"], a["w"], a["lg"], a["cnt"], a["T"],
                                  a["h"], a["E"], a["k"], a["alpha"], a["dt"], a["x"], a["wg"], a["dxin"],
                                  a["dx"], a["dl"], a["dwg"], a["db"], a["ws"], a["wsb"], None)
    assert call(T=-1) == L.MOE_ERR_ARG
    assert call(k=3, E=2) == L.MOE_ERR_ARG
    assert call(E=0) == L.MOE_ERR_SHAPE
    assert call(h=96) == L.MOE_ERR_SHAPE
    assert call(dt=L.MOE_FP8_E4M3) == L.MOE_ERR_DTYPE
    assert call(ypdt=L.MOE_FP8_E4M3) == L.MOE_ERR_DTYPE
    assert call(alpha=float("nan")) == L.MOE_ERR_ARG
    assert call(dwg=None) == L.MOE_ERR_ARG
    assert call(dxin=U) == L.MOE_ERR_ARG
    assert call(dxin=ok["dx"]) == L.MOE_ERR_ARG          # in place is not allowed
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(ws=None) == L.MOE_ERR_WORKSPACE
    assert call(T=0) == L.MOE_OK


def test_router_aux_validation():
    lib = L.lib()
    need = lib.moe_router_aux_workspace_size(1000, 8)
    assert need > 0

    def call(T=1000, E=8, k=2, lg=A, cnt=A, loss=A, ws=A, wsb=need):
        return lib.moe_router_aux_loss(lg, cnt, T, E, k, 0.01, loss, ws, wsb, None)
    assert call(T=0) == L.MOE_ERR_ARG
    assert call(E=L.MOE_MAX_EXPERTS + 1) == L.MOE_ERR_SHAPE
    assert call(k=9) == L.MOE_ERR_ARG
    assert call(loss=None) == L.MOE_ERR_ARG
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE


def test_permute_local_validation():
    lib = L.lib()
    T, h, E, k = 100, 64, 16, 2
    need = lib.moe_permute_local_workspace_size(T, 4, k)
    assert need >= lib.moe_permute_workspace_size(T, 4, k)

    def call(e_lo=4, e_count=4, ws=A, wsb=need, idx=A, dt=L.MOE_BF16):
        return lib.moe_permute_local(A, L.MOE_BF16, idx, None, T, h, E, k, e_lo, e_count, A, A, A, A,
                                     A, dt, None, ws, wsb, None)
    assert call(e_lo=-1) == L.MOE_ERR_ARG
    assert call(e_count=0) == L.MOE_ERR_ARG
    assert call(e_lo=14, e_count=4) == L.MOE_ERR_ARG       # range past E
    assert call(idx=None) == L.MOE_ERR_ARG
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(dt=L.MOE_F32) == L.MOE_ERR_DTYPE


def test_capacity_drop_validation():
    lib = L.lib()
    T, E, k = 100, 8, 2
    need = lib.moe_capacity_drop_workspace_size(T, E, k)
    assert need > 0

    def call(group=2, cap=10, ws=A, wsb=need, T=T, out=A):
        return lib.moe_capacity_drop(A, A, T, E, k, group, cap, out, ws, wsb, None)
    assert call(group=3) == L.MOE_ERR_ARG          # must divide E
    assert call(group=0) == L.MOE_ERR_ARG
    assert call(cap=-1) == L.MOE_ERR_ARG
    assert call(out=None) == L.MOE_ERR_ARG
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(T=0) == L.MOE_OK


def test_grouped_bwd_fp8_validation():
    lib = L.lib()
    need = lib.moe_grouped_bwd_fp8_workspace_size(1000, 256, 384, 8)
    assert need > 0
    Wq = L.MoeWeights(L.MOE_FP8_E4M3, 8, 256, 384, A.value, A.value, A.value, A.value, A.value, A.value,
                      A.value, A.value)
    call = lambda W, ws=A, wsb=need: lib.moe_grouped_swiglu_bwd_fp8(A, A, A, A, A, ctypes.byref(W), A, 1000, A,
                                                                    A, A, A, ws, wsb, None)
    assert call(Wq, wsb=need - 1) == L.MOE_ERR_WORKSPACE
    Wb = L.MoeWeights(L.MOE_BF16, 8, 256, 384, A.value, A.value, None, None, A.value, A.value, None, None)
    assert call(Wb) == L.MOE_ERR_DTYPE
    Wn = L.MoeWeights(L.MOE_FP8_E4M3, 8, 256, 384, A.value, A.value, A.value, A.value, A.value, A.value,
                      None, A.value)
    assert call(Wn) == L.MOE_ERR_ARG


def test_grouped_bwd_fp8_tok_validation():
    """The token-gather FP8 backward rejects bad arguments before any launch."""
    lib = L.lib()
    need = lib.moe_grouped_bwd_fp8_workspace_size(1000, 256, 384, 8)
    Wq = L.MoeWeights(L.MOE_FP8_E4M3, 8, 256, 384, A.value, A.value, A.value, A.value, A.value, A.value,
                      A.value, A.value)

    def call(W=Wq, T=500, k=2, rows=1000, dy=A, x=A, dst_row=A, topk_w=A, ws=A, wsb=need):
        return lib.moe_grouped_swiglu_bwd_fp8_tok(A, A, dy, x, dst_row, topk_w, T, k, A, ctypes.byref(W), A, rows,
                                                  A, A, A, A, ws, wsb, None)
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(rows=1001) == L.MOE_ERR_ARG          # more rows than pairs
    assert call(k=0) == L.MOE_ERR_ARG
    assert call(T=-1) == L.MOE_ERR_ARG
    for name in ("dy", "x", "dst_row", "topk_w"):
        assert call(**{name: None}) == L.MOE_ERR_ARG, name
    Wb = L.MoeWeights(L.MOE_BF16, 8, 256, 384, A.value, A.value, None, None, A.value, A.value, None, None)
    assert call(W=Wb) == L.MOE_ERR_DTYPE


def test_dispatch_swiglu_fwd_validation():
    """The tile-arrival forward rejects bad arguments before any launch."""
    lib = L.lib()
    need = lib.moe_dispatch_swiglu_fwd_workspace_size(500, 2, 256, 384, 8)
    assert need > 0
    Wb = L.MoeWeights(L.MOE_BF16, 8, 256, 384, A.value, A.value, None, None, None, None, None, None)

    def call(W=Wb, T=500, k=2, yp_dtype=L.MOE_BF16, x=A, status=A, ws=A, wsb=need):
        return lib.moe_dispatch_swiglu_fwd(x, A, T, k, A, A, A, A, ctypes.byref(W), A, None, A, yp_dtype, status,
                                           ws, wsb, None)
    assert call(wsb=need - 1) == L.MOE_ERR_WORKSPACE
    assert call(k=0) == L.MOE_ERR_ARG
    assert call(k=9) == L.MOE_ERR_ARG                 # k > E
    assert call(T=-1) == L.MOE_ERR_ARG
    assert call(x=None) == L.MOE_ERR_ARG
    assert call(status=None) == L.MOE_ERR_ARG
    assert call(yp_dtype=L.MOE_FP8_E4M3) == L.MOE_ERR_DTYPE
    Wq = L.MoeWeights(L.MOE_FP8_E4M3, 8, 256, 384, A.value, A.value, A.value, A.value, None, None, None, None)
    assert call(W=Wq) == L.MOE_ERR_DTYPE
    st = lib.moe_dispatch_swiglu_fwd_wait_selftest
    assert st(A, A, 500, 2, A, A, A, A, ctypes.byref(Wb), A, None, A, L.MOE_BF16, A, A, need - 1,
              None) == L.MOE_ERR_WORKSPACE
    assert st(A, A, 500, 2, A, A, A, A, ctypes.byref(Wb), A, None, A, L.MOE_BF16, None, A, need,
              None) == L.MOE_ERR_ARG
