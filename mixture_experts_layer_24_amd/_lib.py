"""ctypes binding of ``libmoe.so`` (the C ABI declared in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_DTYPE = -2
MOE_ERR_SHAPE = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 16

P = ctypes.c_void_p
I = ctypes.c_int
SZ = ctypes.c_size_t
F = ctypes.c_float


class MoeWeights(ctypes.Structure):
    _fields_ = [("dtype", I), ("E", I), ("h", I), ("h_ffn", I),
                ("w13", P), ("w2", P), ("w13_scale", P), ("w2_scale", P),
                ("w13_bwd", P), ("w2_bwd", P), ("w13_bwd_scale", P), ("w2_bwd_scale", P)]


SIGNATURES = {
    "moe_packed_weight_bytes": (SZ, [I, I, I, I, I]),
    "moe_pack_weights": (I, [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P]),
    "moe_route": (I, [P, P, P, P, I, I, I, I, I, P, P, P]),
    "moe_permute_workspace_size": (SZ, [I, I, I]),
    "moe_permute": (I, [P, I, P, P, I, I, I, I, P, P, P, P, P, I, P, P, SZ, P]),
    "moe_permute_noalloc": (I, [P, I, P, P, I, I, I, I, P, P, P, P, P, I, P, P]),
    "moe_permute_local_workspace_size": (SZ, [I, I, I]),
    "moe_permute_local": (I, [P, I, P, P, I, I, I, I, I, I, P, P, P, P, P, I, P, P, SZ, P]),
    "moe_capacity_drop_workspace_size": (SZ, [I, I, I]),
    "moe_capacity_drop": (I, [P, P, I, I, I, I, I, P, P, SZ, P]),
    "moe_grouped_workspace_size": (SZ, [I, I, I, I, I]),
    "moe_grouped_swiglu_fwd": (I, [P, P, ctypes.POINTER(MoeWeights), P, I, P, P, I, P, SZ, P]),
    "moe_grouped_bwd_workspace_size": (SZ, [I, I, I, I, I]),
    "moe_grouped_swiglu_bwd": (I, [P, P, P, ctypes.POINTER(MoeWeights), P, I, P, P, P, P, P, SZ, P]),
    "moe_combine": (I, [P, I, P, P, I, I, I, P, I, P]),
    "moe_grouped_bwd_fp8_workspace_size": (SZ, [I, I, I, I]),
    "moe_grouped_swiglu_bwd_fp8": (I, [P, P, P, P, P, ctypes.POINTER(MoeWeights), P, I, P, P, P, P, P, SZ, P]),
    "moe_grouped_swiglu_bwd_fp8_tok": (I, [P, P, P, P, P, P, I, I, P, ctypes.POINTER(MoeWeights), P, I, P, P, P,
                                           P, P, SZ, P]),
    "moe_dispatch_swiglu_fwd_workspace_size": (SZ, [I, I, I, I, I]),
    "moe_dispatch_swiglu_fwd": (I, [P, P, I, I, P, P, P, P, ctypes.POINTER(MoeWeights), P, P, P, I, P, P, SZ, P]),
    "moe_dispatch_swiglu_fwd_wait_selftest": (I, [P, P, I, I, P, P, P, P, ctypes.POINTER(MoeWeights), P, P, P, I, P, P, SZ, P]),
    "moe_router_bwd_workspace_size": (SZ, [I, I, I]),
    "moe_router_bwd": (I, [P, P, I, P, P, P, P, P, I, I, I, I, F, I, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_router_aux_workspace_size": (SZ, [I, I]),
    "moe_router_aux_loss": (I, [P, P, I, I, I, F, P, P, SZ, P]),
    "moe_timing_enable": (I, [I]),
    "moe_timing_report": (I, [ctypes.c_char_p, SZ]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (I, []),
    "moe_fp8_convert_selftest": (I, [P, P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_24_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def check(rc: int) -> int:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc
