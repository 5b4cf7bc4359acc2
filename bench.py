#!/usr/bin/env python3
"""Throughput of the LittleBit linear forward on one MI355X.

One step = one forward sweep of the whole workload (every matrix of the
stack, chained as a transformer would chain them) on one batch of
synthetic input already resident in HBM.  The default workload is the
Llama2-70B MLP stack at 0.1 bits per weight with the residual path
(80 blocks x gate, up 8192->28672 and down 28672->8192, rank 302, M = 1).

Prints one JSON line.  value = algorithmic bytes of one sweep (sign bits,
fp16 scales, fp16 activations in and out of every matrix) / time per
step, in GB/s.  The oracle (float64 numpy) is timed on the host cores on
a bounded sample of the same workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lb_synth  # noqa: E402

METRIC = ("LittleBit linear fwd: µs/layer + achieved HBM GB/s vs 8 TB/s at batch 1; "
          "M=128 TFLOP/s")
HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(wl: dict, M: int) -> int:
    tot = 0
    for sp in wl["layers"]:
        P = 2 if sp["residual"] else 1
        a, b, s = sp["a"], sp["b"], sp["s"]
        tot += P * s * (a + b) // 8          # sign bits (P*s*(a+b) is a multiple of 8 here)
        tot += 2 * P * (a + b + s)           # fp16 h, g, l
        tot += 2 * M * (a + b)               # fp16 input and output rows
    return tot


def algorithmic_flops(wl: dict, M: int) -> int:
    tot = 0
    for sp in wl["layers"]:
        P = 2 if sp["residual"] else 1
        tot += 2 * M * P * sp["s"] * (sp["a"] + sp["b"])
    return tot


def build(lbm, wl):
    layers, t0 = [], time.time()
    for sp in wl["layers"]:
        layers.append(lbm.Layer.from_paths(lb_synth.workload_layer_inputs(sp)))
    P = 2 if wl["layers"][0]["residual"] else 1
    stack = lbm.Stack(layers, wl["units"], lb_synth.kappa(P))
    return stack, time.time() - t0


def time_steps(torch, stack, x, y, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        stack.forward(x, y, None, stream=stream)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        stack.forward(x, y, None, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall / steps * 1e3


KERNEL_SRC = {"persistent": "binary_rank_gemv_littlebitlinear_amd/csrc/lb_persist.hip",
              "unit": "binary_rank_gemv_littlebitlinear_amd/csrc/lb_mfma.hip"}


def kernel_hash(kind: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SRC[kind]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, kind: str, blocks):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the same
    counters on a copy of known size), or None when there is no summary for
    this workload or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_hash(kind) or t.get("blocks") != blocks:
        return None
    return t.get("hbm_bytes_per_launch")


def copy_probe(torch, mib: int):
    """An elementwise kernel of known size (reads and writes MIB MiB each;
    calibrates the HBM byte counters)."""
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: 3 x neg over {mib} MiB", file=sys.stderr, flush=True)


def cpu_baseline(wl: dict, M: int, budget_s: float) -> dict:
    """Time the float64 oracle on a bounded sample of the workload's layers."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    x = lb_synth.activations(M, wl["layers"][0]["a"], seed=wl["seed"])
    done_bytes, done_layers, t_used = 0, 0, 0.0
    one = {"layers": None}
    for sp in wl["layers"]:
        paths = lb_synth.workload_layer_inputs(sp)
        xin = x if x.shape[1] == sp["a"] else lb_synth.activations(M, sp["a"], seed=sp["block"])
        t0 = time.perf_counter()
        oracle.forward(xin, paths)
        t_used += time.perf_counter() - t0
        one["layers"] = [sp]
        done_bytes += algorithmic_bytes(one, M)
        done_layers += 1
        if t_used >= budget_s:
            break
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done_layers} of {len(wl['layers'])} matrices, M={M}, "
                      f"float64 numpy incl. bit unpack, {t_used:.1f} s"}


def init_cpu_baseline(U, V) -> dict:
    """The oracle's initialisation (one call) and Joint-ITQ (5 steps, scaled
    to 50: every step costs the same) on the same factors, on the host."""
    import oracle
    t0 = time.perf_counter()
    oracle.init_from_factors(U, V)
    init_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.joint_itq_rotation(U, V, 5)
    itq5_s = time.perf_counter() - t0
    return {"init_ms": round(init_s * 1e3, 1), "joint_itq_50_ms": round(itq5_s * 10 * 1e3, 1),
            "kind": "oracle", "sample": "one init call; Joint-ITQ timed over 5 steps x 10"}


def measure_init(torch, lbm, reps: int = 3, with_cpu: bool = False) -> dict:
    """Initialisation of one Llama2-70B gate projection (8192 -> 28672, rank
    302) from real fp32 factors already on the device: wall time of the
    synchronous lb_init_from_factors call (sign packing, the two rank-1
    fits, scales and the device re-layout of the result), of lb_joint_itq
    with 50 steps, and of lb_init_from_factors from the rotated factors."""
    a, b, s = 8192, 28672, 302
    U, V = lb_synth.factors(a, b, s, seed=3)
    Ud, Vd = torch.from_numpy(U).cuda(), torch.from_numpy(V).cuda()
    L = lbm.Layer(a, b, s, True)
    lbm.lb_init_from_factors(L.handle, 0, Ud, Vd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(reps):
        lbm.lb_init_from_factors(L.handle, i % 2, Ud, Vd)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    # Joint-ITQ (50 steps, the pages' default) and the path from the rotated factors
    R = lbm.lb_joint_itq(Ud, Vd, 50)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        R = lbm.lb_joint_itq(Ud, Vd, 50)
    torch.cuda.synchronize()
    itq_ms = (time.perf_counter() - t0) * 1e3 / reps
    t0 = time.perf_counter()
    for i in range(reps):
        lbm.lb_init_from_factors(L.handle, i % 2, Ud, Vd, R)
    torch.cuda.synchronize()
    rot_ms = (time.perf_counter() - t0) * 1e3 / reps
    L.close()
    n = a + b
    itq_flops = 50 * 4 * n * s * s  # X R and X^T B per step (Newton-Schulz products not counted)
    out = {"layer": "llama70b gate 8192->28672", "s": s, "ms_per_call": round(ms, 3),
           "factor_bytes": (a + b) * s * 4, "joint_itq_50_ms": round(itq_ms, 3),
           "joint_itq_gemm_tflops": round(itq_flops / (itq_ms * 1e-3) / 1e12, 3),
           "init_rotated_ms": round(rot_ms, 3)}
    if with_cpu:
        out["cpu_baseline"] = init_cpu_baseline(U, V)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_mlp_stack", choices=sorted(lb_synth.WORKLOADS))
    ap.add_argument("--blocks", type=int, default=None)
    ap.add_argument("--rows", type=int, default=None,
                    help="override the workload's token count M (small-batch measurements)")
    ap.add_argument("--mode", type=int, default=0, help="0 auto, 1 per-layer kernels, 2 persistent")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", default="llama7b_full_stack_M128",
                    help="extra workload measured in the same run ('' to skip)")
    ap.add_argument("--no-init", action="store_true",
                    help="skip timing the initialisation from real factors")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not part of this benchmark.", file=sys.stderr)
        sys.exit(2)

    import torch
    import binary_rank_gemv_littlebitlinear_amd as lbm
    assert torch.cuda.is_available(), "no GPU visible"
    lbm.load_library()

    def measure(name, blocks, with_cpu):
        wl = lb_synth.workload(name, blocks)
        if args.rows is not None and name == args.workload:
            wl["M"] = int(args.rows)
        M = wl["M"]
        print(f"[bench] building {name} ({len(wl['layers'])} matrices, M={M})", file=sys.stderr, flush=True)
        stack, t_build = build(lbm, wl)
        stack.set_mode(args.mode)
        stack.reserve(M)
        x = torch.from_numpy(lb_synth.activations(M, wl["layers"][0]["a"], seed=wl["seed"])).cuda()
        y = torch.empty((M, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
        print(f"[bench] built in {t_build:.1f} s; timing {args.steps} steps", file=sys.stderr, flush=True)
        ms, wall_ms = time_steps(torch, stack, x, y, args.steps, args.warmup)
        nbytes, flops = algorithmic_bytes(wl, M), algorithmic_flops(wl, M)
        res = {"wl": wl, "M": M, "ms": ms, "wall_ms": wall_ms, "bytes": nbytes, "flops": flops}
        if with_cpu:
            print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
            res["cpu"] = cpu_baseline(wl, M, args.cpu_budget)
        stack.close()
        torch.cuda.synchronize()
        return res

    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
    r = measure(args.workload, args.blocks, not args.no_cpu_baseline)
    wl, M, ms = r["wl"], r["M"], r["ms"]
    gbs = r["bytes"] / (ms * 1e-3) / 1e9
    tflops = r["flops"] / (ms * 1e-3) / 1e12
    batch1 = M < 64
    kind = "persistent" if (M <= 1 and args.mode != 1) else "unit"
    traffic = measured_traffic(wl["name"], kind, wl["blocks"]) if kind == "persistent" else None
    out = {
        "metric": METRIC,
        "value": round(gbs if batch1 else tflops, 3),
        "unit": "GB/s" if batch1 else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl["name"], "M": M, "blocks": wl["blocks"],
                   "matrices": len(wl["layers"]), "s": sorted({sp["s"] for sp in wl["layers"]}),
                   "residual": wl["layers"][0]["residual"], "parallelism": "single GPU"},
        "us_per_layer": round(ms * 1e3 / wl["blocks"], 4),
        "tokens_per_s_equiv": round(M / (ms * 1e-3), 1),
        "algorithmic_bytes_per_step": r["bytes"],
        "roofline": {"bound": "hbm" if batch1 else "mfma",
                     "achieved": round(gbs if batch1 else tflops, 3),
                     "peak": HBM_PEAK_GBS if batch1 else MFMA_FP16_PEAK_TFLOPS,
                     "unit": "GB/s" if batch1 else "TFLOP/s",
                     "frac": round((gbs / HBM_PEAK_GBS) if batch1 else (tflops / MFMA_FP16_PEAK_TFLOPS), 4),
                     "traffic": traffic,
                     "kernel": ("k_persist: one launch per step, timed with events on its stream"
                                if kind == "persistent" else
                                "k_unit_s1 + k_unit_s2 per unit, timed together with events on their stream")},
    }
    if "cpu" in r:
        out["cpu_baseline"] = r["cpu"]
    if args.secondary and args.secondary != args.workload:
        s2 = measure(args.secondary, None, False)
        ms2 = s2["ms"]
        out["secondary"] = {"workload": args.secondary, "M": s2["M"], "ms_per_step": round(ms2, 5),
                            "us_per_layer": round(ms2 * 1e3 / s2["wl"]["blocks"], 3),
                            "TFLOP/s": round(s2["flops"] / (ms2 * 1e-3) / 1e12, 3),
                            "mfma_frac": round(s2["flops"] / (ms2 * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                            "GB/s": round(s2["bytes"] / (ms2 * 1e-3) / 1e9, 2),
                            "tokens_per_s_equiv": round(s2["M"] / (ms2 * 1e-3), 1)}
    if not args.no_init:
        print("[bench] timing initialisation from real factors", file=sys.stderr, flush=True)
        out["init"] = measure_init(torch, lbm, with_cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
