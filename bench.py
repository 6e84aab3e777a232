#!/usr/bin/env python3
"""Benchmark one MoE expert layer step on one MI355X.

A step is the whole hot path on one batch: route (gate GEMM + top-k softmax)
-> dispatch (index build + permute) -> grouped SwiGLU GEMMs -> weighted
combine, plus, for workloads that train, the load-balance loss and the backward
(experts and router).  Inputs are seeded,
synthetic and already resident in HBM when the timed region starts; weights
are packed once before it.

Prints ONE JSON line (see the repository's design notes for every field).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12}   # dense MFMA FLOP/s, MI355X
HBM_PEAK = 8.0e12                                          # B/s
METRIC = "MoE layer tokens/s and GroupedGEMM TFLOP/s (% of MFMA peak) on 1 MI355X"
AUX_ALPHA = 0.01  # weight of the load-balance loss in training steps


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_engine.h", "gemm_fwd.hip"):
        with open(os.path.join(ROOT, "mixture_experts_layer_24_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, kernel: str):
    """Bytes per launch of `kernel` read and written beyond L2 (scaled
    FETCH_SIZE + WRITE_SIZE, which include Infinity Cache hits) from the
    committed counter profile, or None when there is none or the GEMM sources
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_fwd.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    k = t.get("kernels", {}).get(kernel)
    if k is None or t.get("source_sha") != gemm_source_sha():
        return None
    return (k["read_bytes"] + k["write_bytes"]) / 1e9


def cpu_baseline(wl, inp, n_tokens, seed=0):
    """Time the CPU oracle on the first n_tokens tokens of the same batch."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from moe_synth import to_f32
    from oracle import moe_ref as ref

    class PerExpert:
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __getitem__(self, e):
            return to_f32(self.a[e])

    x = to_f32(inp["x"][:n_tokens])
    wg = to_f32(inp["w_gate"])
    w1, w3, w2 = PerExpert(inp["w1"]), PerExpert(inp["w3"]), PerExpert(inp["w2"])
    t0 = time.perf_counter()
    if wl.dtype == "fp8":
        out = ref.layer_forward_fp8(x, wg, inp["bias"], w1, w3, w2, wl.k)
        if wl.backward:
            dy = to_f32(inp["dy"][:n_tokens])
            ref.aux_balance_loss(out["logits"], out["idx"], wl.E, wl.k, AUX_ALPHA)
            ref.layer_backward_fp8(dy, x, out["w"], out["dst_row"], out["offsets"], w1, w3, w2,
                                   out["g"], out["u"])
            ref.router_backward(dy, out["yp"][out["dst_row"]], x, wg, out["logits"], out["idx"],
                                out["w"], AUX_ALPHA)
    else:
        out = ref.layer_forward(x, wg, inp["bias"], w1, w3, w2, wl.k)
        if wl.backward:
            dy = to_f32(inp["dy"][:n_tokens])
            ref.aux_balance_loss(out["logits"], out["idx"], wl.E, wl.k, AUX_ALPHA)
            ref.layer_backward(dy, x, out["w"], out["dst_row"], out["offsets"], w1, w3, w2,
                               g=out["g"], u=out["u"])
            ref.router_backward(dy, out["yp"][out["dst_row"]], x, wg, out["logits"], out["idx"],
                                out["w"], AUX_ALPHA)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu, "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"first {n_tokens} of {wl.T} tokens of the same seeded batch, full layer "
                      f"{'fwd+bwd' if wl.backward else 'fwd'} in fp64 NumPy ({dt:.1f} s)"}


# Workloads timed beside the primary one when bench.py runs without --workload
# (each a shape from the pages' model table; see moe_synth.WORKLOADS).
OTHER_WORKLOADS = ("dsmoe", "dsmoe_fp8", "hunyuan_fp8", "m352b_zipf", "mixtral22b", "phi35")


def measure(name, steps, warmup, cold, arrival=False):
    """Generate one workload's inputs, time `steps` layer steps after `warmup`
    untimed ones, and return (the JSON fields, the workload, its host inputs).
    With `arrival` (BF16 workloads) the layer overlaps its dispatch copy and
    FC1 by tile arrival (moe_dispatch_swiglu_fwd)."""
    import numpy as np
    import torch

    import moe_synth
    from mixture_experts_layer_24_amd import accounting as acc
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16, MOE_F32, MOE_FP8_E4M3

    wl = moe_synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"bench: generating {wl.name} inputs")
    inp = moe_synth.gen_all(wl, seed=0)

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    code = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}[wl.dtype]
    x, wg, bias = t(inp["x"]), t(inp["w_gate"]), torch.from_numpy(inp["bias"]).to(dev)
    w1, w3, w2 = t(inp["w1"]), t(inp["w3"]), t(inp["w2"])
    P = ops.PackedWeights(w1, w3, w2, code, backward=wl.backward)
    del w1, w3, w2
    layer = ops.MoELayer(wl.T, wl.h, wl.h_ffn, wl.E, wl.k, code, device=dev,
                         save_for_backward=wl.backward)
    dy = t(inp["dy"]) if wl.backward else None

    def step():
        layer.forward(x, wg, bias, P, arrival=arrival)
        if wl.backward:
            layer.aux_loss(AUX_ALPHA)
            layer.backward(dy, x, P, w_gate=wg, alpha=AUX_ALPHA)

    log(f"bench: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {steps} steps")
    ops.moe_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern = ops.moe_timing_report()
    ops.moe_timing_enable(False)
    ms = elapsed * 1e3 / steps

    # Figures beside `value`: per-step times (events around each step) warm,
    # and cold: a 1 GiB read-modify-write before each step evicts L2 and the
    # 256 MB Infinity Cache (outside the events).
    def timed_steps(n, flush=None):
        ts = []
        for _ in range(n):
            if flush is not None:
                flush.add_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)

    log("bench: per-step" + (" and cold-cache steps" if cold else " times"))
    warm = timed_steps(steps)
    if cold:
        flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        cold_ts = timed_steps(min(steps, 5), flush_buf)
        del flush_buf
    step_stats = lambda ts: {"median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4), "n": len(ts)}
    # GEMM bound per expert: max(FLOPs / peak, weight bytes / HBM), summed (forward)
    attainable = None
    if not wl.backward:
        cnt = layer.counts.cpu().tolist()
        wbytes = 3 * wl.h * wl.h_ffn * (1 if wl.dtype == "fp8" else 4 if wl.dtype == "f32" else 2)
        attainable = sum(max(6.0 * m * wl.h * wl.h_ffn / PEAK[wl.dtype], wbytes / HBM_PEAK) for m in cnt) * 1e3
    counts = acc.workload_counts(wl)
    avg = {k: v[1] / v[0] for k, v in kern.items()}          # ms per launch
    per_step = {k: v[1] / steps for k, v in kern.items()}
    flops_step = counts["flops_fwd"] + counts.get("flops_bwd", 0)
    gemm_ms = sum(per_step.get(k, 0.0) for k in ("fc1", "fc2", "bwd_dA", "bwd_dW2", "bwd_dXp", "bwd_dW13"))
    peak = PEAK[wl.dtype]
    gemm_tflops = flops_step / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None

    dom = max(per_step, key=per_step.get)
    flops_per_launch = {"fc1": counts["flops_fc1"], "fc2": counts["flops_fc2"]}
    if wl.backward:
        rhf = wl.R * wl.h * wl.h_ffn
        flops_per_launch.update(bwd_dA=2 * rhf, bwd_dW2=2 * rhf, bwd_dXp=4 * rhf, bwd_dW13=4 * rhf)
    # mean algorithmic bytes per launch over the step's launches of each kernel
    # (a training step dispatches x, dY (and its FP8 codes) and re-gathers x;
    # its second combine writes the expert path's dX in fp32)
    mean = lambda v: sum(v) / len(v)
    bytes_per_launch = {"permute": mean(counts["permute_launches"]),
                        "combine": mean(counts["combine_launches"]),
                        "route": counts["router_bytes"]}
    if dom in flops_per_launch:
        achieved = flops_per_launch[dom] / (avg[dom] * 1e-3)
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None}
    else:
        achieved = bytes_per_launch.get(dom, 0) / (avg[dom] * 1e-3)
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": achieved / HBM_PEAK, "traffic": None}
    roof["traffic"] = profiled_traffic(wl.name, dom)
    roof["traffic_unit"] = ("GB per launch read and written beyond L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated; Infinity Cache hits included)")
    roof["time_source"] = ("mean launch time of the kernel over the timed steps, HIP events recorded on the "
                           "launch stream around each launch")
    hbm = {}
    for k2, b in bytes_per_launch.items():
        if k2 in avg:
            bw = b / (avg[k2] * 1e-3)
            hbm[k2] = {"GB/s": round(bw / 1e9, 1), "frac": round(bw / HBM_PEAK, 4)}
    out = {
        "metric": METRIC, "value": wl.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} MoE layer {'fwd+bwd' if wl.backward else 'fwd'}",
                   "T": wl.T, "h": wl.h, "h_ffn": wl.h_ffn, "E": wl.E, "k": wl.k,
                   **({"dispatch": "tile arrival (copy and FC1 overlapped)"} if arrival else {})},
        "gemm_tflops": gemm_tflops, "gemm_frac_of_peak": (gemm_tflops * 1e12 / peak) if gemm_tflops else None,
        "kernel_ms_per_step": {k: round(v, 4) for k, v in per_step.items()},
        "hbm": hbm,
        "roofline": roof,
        "step_ms": step_stats(warm),
    }
    if cold:
        out["cold_step_ms"] = dict(step_stats(cold_ts), flush_bytes=1 << 30)
    if attainable is not None:
        out["gemm_attainable_ms"] = round(attainable, 4)
    del P, layer, x, wg, bias, dy
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out, wl, inp


def moe_synth_dtype(name):
    import moe_synth
    return moe_synth.WORKLOADS[name].dtype


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: mixtral, then the other shapes as `other_workloads`)")
    ap.add_argument("--arrival", action="store_true",
                    help="with --workload (BF16): overlap the dispatch copy and FC1 by tile arrival")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="most tokens in the CPU oracle sample, kept under ~45 s (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (3 times), to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU layout is a design in the notes, not built here.", file=sys.stderr)
        sys.exit(2)

    primary = args.workload or "mixtral"
    if args.arrival and (args.workload is None or moe_synth_dtype(primary) != "bf16"):
        print("--arrival needs --workload with a BF16 workload", file=sys.stderr)
        sys.exit(2)
    out, wl, inp = measure(primary, args.steps, args.warmup, cold=True, arrival=args.arrival)
    if args.workload is None:
        # the other workloads of the same build, timed in the same run with the
        # same step counts (no cold-cache pass): figures beside `value`
        others = {}
        for name in OTHER_WORKLOADS:
            o, _, _ = measure(name, args.steps, args.warmup, cold=False)
            others[name] = {k: o[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                              "gemm_tflops", "gemm_frac_of_peak", "roofline",
                                              "hbm", "kernel_ms_per_step", "step_ms")}
            others[name]["roofline"] = {k: o["roofline"][k]
                                        for k in ("kernel", "bound", "achieved", "peak", "unit", "frac")}
            if "gemm_attainable_ms" in o:
                others[name]["gemm_attainable_ms"] = o["gemm_attainable_ms"]
        out["other_workloads"] = others
    if args.cpu_tokens > 0:
        # a short probe bounds the sample: the oracle's time grows at most
        # linearly in tokens (it has a fixed per-expert part), so the whole
        # requested sample runs unless the probe extrapolates past ~45 s
        n0 = min(512, args.cpu_tokens, wl.T)
        probe = cpu_baseline(wl, inp, n0)
        n = min(args.cpu_tokens, wl.T)
        if n0 / probe["value"] * n / n0 > 45.0:
            n = int(max(n0, 45.0 * probe["value"]))
        log(f"bench: cpu oracle on {n} tokens")
        out["cpu_baseline"] = cpu_baseline(wl, inp, n) if n > 512 else probe
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
