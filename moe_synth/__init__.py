"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the CPU oracle and the GPU path: it produces input
tensors only and holds none of the layer's arithmetic.  Every tensor is drawn
from ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, chunk])))``
so a chunk (one expert's weight matrix, or one block of token rows) can be
generated on its own, in parallel, or sampled without generating the rest.

Storage forms
-------------
* fp32 workloads: ``numpy.float32`` arrays.
* bf16 workloads: ``numpy.uint16`` arrays holding bf16 bit patterns (values are
  drawn in fp32 then rounded to nearest-even bf16).  ``bf16_bits_to_f32``
  widens them exactly.

Shapes (row-vector convention ``y = x @ W``)
-------------------------------------------
x ``[T, h]``, router ``w_gate`` ``[h, E]``, ``bias`` ``[E]`` fp32 (zeros unless
the workload is skewed), expert ``w1``/``w3`` ``[E, h, h_ffn]`` (gate / up),
``w2`` ``[E, h_ffn, h]`` (down), upstream gradient ``dy`` ``[T, h]``.

Workload shapes come from the model-shape table of the MegaScale-MoE pages
(paper review, section 五 "基准测试配置"; research digest, Table 2 shapes):
Mixtral-8x7B, DeepSeekMoE, Internal-352B, Hunyuan-Large, Mixtral-8x22B and
Phi-3.5-MoE (the table gives no batch; the last two use the Mixtral batch).  The value
distributions (N(0,1) activations, N(0, 1/fan_in) expert weights, N(0, 0.02)
router, Zipf(1.2) router bias for the skewed workload) are this project's
synthetic stand-ins: the pages publish no weights or data.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"x": 1, "w_gate": 2, "w1": 3, "w3": 4, "w2": 5, "dy": 6,
              # stand-ins for intermediate tensors when one step is tested alone
              "yp": 7, "dx_in": 8}
ROW_CHUNK = 1024  # token rows per generator stream for x and dy


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    h: int
    h_ffn: int
    E: int
    k: int
    dtype: str            # "f32", "bf16" or "fp8" (fp8: bf16 storage, fp8 compute)
    backward: bool = False
    zipf_s: float = 0.0   # >0: router bias = log of Zipf(s) expert weights
    router_std: float = 0.02

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def storage(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 256, 512, 8, 2, "f32"),
    "mixtral": Workload("mixtral", 8192, 4096, 14336, 8, 2, "bf16"),
    "dsmoe": Workload("dsmoe", 16384, 2048, 1408, 64, 6, "bf16", backward=True),
    "m352b_zipf": Workload("m352b_zipf", 8192, 4096, 14336, 32, 3, "bf16", zipf_s=1.2),
    "hunyuan_fp8": Workload("hunyuan_fp8", 32768, 6400, 18304, 16, 1, "fp8"),
    # the two remaining shapes of the model table, at the Mixtral batch
    "mixtral22b": Workload("mixtral22b", 8192, 6144, 16384, 8, 2, "bf16"),
    "phi35": Workload("phi35", 8192, 4096, 6400, 16, 2, "bf16"),
    # the DeepSeekMoE-shaped training step with per-token FP8 in both passes
    "dsmoe_fp8": Workload("dsmoe_fp8", 16384, 2048, 1408, 64, 6, "fp8", backward=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tensor: str, chunk: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, TENSOR_IDS[tensor], chunk])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(a: np.ndarray) -> np.ndarray:
    """Storage form (fp32 or bf16 bits) -> fp32 values."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def _normal(seed, tensor, chunk, shape, std, storage):
    v = _rng(seed, tensor, chunk).standard_normal(int(np.prod(shape)), dtype=np.float32)
    v *= np.float32(std)
    v = v.reshape(shape)
    return f32_to_bf16_bits(v) if storage == "bf16" else v


def gen_matrix(tensor: str, shape, std: float = 1.0, storage: str = "bf16", seed: int = 0) -> np.ndarray:
    """A whole N(0, std^2) tensor from one stream (small test inputs)."""
    return _normal(seed, tensor, 0, tuple(shape), std, storage)


def gen_rows(wl: Workload, tensor: str, rows: np.ndarray, seed: int = 0) -> np.ndarray:
    """Rows ``rows`` of the token-major tensor ``tensor`` ("x" or "dy")."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), wl.h), dtype=np.uint16 if wl.storage == "bf16" else np.float32)
    for c in np.unique(rows // ROW_CHUNK):
        n = min(ROW_CHUNK, wl.T - c * ROW_CHUNK)
        blk = _normal(seed, tensor, int(c), (n, wl.h), 1.0, wl.storage)
        sel = np.nonzero(rows // ROW_CHUNK == c)[0]
        out[sel] = blk[rows[sel] - c * ROW_CHUNK]
    return out


def gen_tokens(wl: Workload, tensor: str = "x", seed: int = 0) -> np.ndarray:
    nchunks = (wl.T + ROW_CHUNK - 1) // ROW_CHUNK
    dt = np.uint16 if wl.storage == "bf16" else np.float32
    out = np.empty((wl.T, wl.h), dtype=dt)

    def one(c):
        n = min(ROW_CHUNK, wl.T - c * ROW_CHUNK)
        out[c * ROW_CHUNK:c * ROW_CHUNK + n] = _normal(seed, tensor, c, (n, wl.h), 1.0, wl.storage)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nchunks)))
    return out


def gen_router(wl: Workload, seed: int = 0):
    """Router weight ``[h, E]`` (storage form) and bias ``[E]`` fp32.

    The skewed workload's bias is ``log p_e`` with ``p_e`` proportional to
    ``(e+1)^-s`` (expert 0 is the most popular), added to the logits.
    """
    wg = _normal(seed, "w_gate", 0, (wl.h, wl.E), wl.router_std, wl.storage)
    if wl.zipf_s > 0:
        r = np.arange(1, wl.E + 1, dtype=np.float64) ** (-wl.zipf_s)
        bias = np.log(r / r.sum()).astype(np.float32)
    else:
        bias = np.zeros(wl.E, dtype=np.float32)
    return wg, bias


def gen_expert(wl: Workload, e: int, seed: int = 0):
    """Expert ``e``'s (w1 [h,h_ffn], w3 [h,h_ffn], w2 [h_ffn,h]) in storage form."""
    s13 = 1.0 / math.sqrt(wl.h)
    s2 = 1.0 / math.sqrt(wl.h_ffn)
    w1 = _normal(seed, "w1", e, (wl.h, wl.h_ffn), s13, wl.storage)
    w3 = _normal(seed, "w3", e, (wl.h, wl.h_ffn), s13, wl.storage)
    w2 = _normal(seed, "w2", e, (wl.h_ffn, wl.h), s2, wl.storage)
    return w1, w3, w2


def gen_experts(wl: Workload, seed: int = 0):
    """All experts' weights, stacked ``[E, ...]`` in storage form."""
    dt = np.uint16 if wl.storage == "bf16" else np.float32
    w1 = np.empty((wl.E, wl.h, wl.h_ffn), dtype=dt)
    w3 = np.empty_like(w1)
    w2 = np.empty((wl.E, wl.h_ffn, wl.h), dtype=dt)

    def one(job):
        e, name = job
        std = 1.0 / math.sqrt(wl.h if name != "w2" else wl.h_ffn)
        shape = (wl.h_ffn, wl.h) if name == "w2" else (wl.h, wl.h_ffn)
        {"w1": w1, "w3": w3, "w2": w2}[name][e] = _normal(seed, name, e, shape, std, wl.storage)

    jobs = [(e, n) for e in range(wl.E) for n in ("w1", "w3", "w2")]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, jobs))
    return w1, w3, w2


def gen_all(wl: Workload, seed: int = 0) -> dict:
    """Every input of one layer call, in storage form."""
    x = gen_tokens(wl, "x", seed)
    wg, bias = gen_router(wl, seed)
    w1, w3, w2 = gen_experts(wl, seed)
    out = dict(x=x, w_gate=wg, bias=bias, w1=w1, w3=w3, w2=w2)
    if wl.backward:
        out["dy"] = gen_tokens(wl, "dy", seed)
    return out
