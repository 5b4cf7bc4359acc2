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
MALL_BYTES = 256 << 20
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


def kernel_desc(M: int, mode: int) -> str:
    """The kernels lb_stack_forward runs for M rows in this mode (no trace)."""
    if M <= 1 and mode != 1:
        return "k_persist: one launch per step, timed with events on its stream"
    if M == 2 and mode in (0, 3):
        return "k_persist once per row, timed with events on its stream"
    if M >= 3 and mode in (0, 3):
        return "k_mstack: one launch per 256 rows, timed with events on its stream"
    if M >= 64:
        return "k_unit_s1 + k_unit_s2 per unit, timed together with events on their stream"
    return "wave-path kernels per layer, timed together with events on their stream"


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


def mall_reference(torch, nbytes: int, reps: int = 50) -> dict:
    """Read bandwidth of a buffer of the workload's own size when it fits the
    256 MB MALL: torch's sum over an fp16 buffer of ``nbytes``, read ``reps``
    times after a warm-up (the first pass brings it in; later passes read it
    from the MALL).  The reference the stack's algorithmic GB/s is set
    against for a MALL-resident working set."""
    n = nbytes // 2
    buf = torch.ones(n, dtype=torch.float16, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(5):
        torch.sum(buf, dim=0, dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.sum(buf, dim=0, dtype=torch.float32, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"buffer_bytes": 2 * n, "read_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "kernel": "torch.sum over the buffer, fp16 read, fp32 accumulate",
            "reps": reps}


TIMELINE_PARTS = ("second-product lookups", "second-product epilogue, combine and next tables",
                  "first-product set-up", "first-product lookups and publish",
                  "barrier + level A (XCD-local sum)", "level B (across XCDs)", "level C + next tables")


def sweep_timeline(torch, lbm, stack, x, y, nunits: int) -> dict:
    """Where a phase of the one-launch sweep spends its time: one sweep with
    lb_stack_timeline's device timestamps (eight per phase and workgroup,
    100 MHz), medians over workgroups and over the phases of each kind
    (odd phases carry the gate/up second product and the down first product,
    even ones the reverse)."""
    need = lbm.lb_stack_timeline(stack.handle, None, 0)
    buf = torch.zeros(need, dtype=torch.int64, device="cuda")
    lbm.lb_stack_timeline(stack.handle, buf, need)
    stack.forward(x, y)
    torch.cuda.synchronize()
    lbm.lb_stack_timeline(stack.handle, None, 0)
    stack.check()
    G = need // ((nunits + 1) * 8)
    t = buf.cpu().numpy().reshape(G, nunits + 1, 8).astype(np.int64)
    out = {"workgroups": int(G), "phases": nunits + 1}
    for kind, sel in (("heavy", list(range(1, nunits, 2))), ("light", list(range(2, nunits, 2)))):
        if not sel:
            continue
        parts = {n: round(float(np.median(t[:, sel, k + 1] - t[:, sel, k])) / 100.0, 3)
                 for k, n in enumerate(TIMELINE_PARTS)}
        period = float(np.median(np.diff(t[:, :, 0], axis=1)[:, sel])) / 100.0  # start to next start
        out[kind + "_phase_us"] = parts
        out[kind + "_exchange_us"] = round(sum(parts[n] for n in TIMELINE_PARTS[4:]), 3)
        out[kind + "_period_us"] = round(period, 3)
    return out


def _time_eager(torch, fn, reps: int) -> float:
    """ms per call of fn, events on torch's current stream after warm-up."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def dense_fp16_reference(torch, wl: dict, M: int, ours_ms: float, max_gib: float = 16.0,
                         reps: int = 10) -> dict:
    """The FP16 baseline of the pages' speed-up figure, on this GPU: the same
    stack wiring with dense fp16 weights (b x a per matrix, random: timing
    only) through torch's linear (the platform's GEMV/GEMM library).  Only the
    first blocks that fit max_gib are built; each is distinct, and a block's
    time is bound by streaming its weights, so their mean per-block time
    stands for the whole stack.  Context, not a target."""
    F = torch.nn.functional
    per = wl["per_block"]
    ub = wl["units"][:len(wl["units"]) // wl["blocks"]]
    blk_bytes = sum(2 * sp["a"] * sp["b"] for sp in wl["layers"][:per])
    nb = max(1, min(wl["blocks"], int(max_gib * (1 << 30)) // blk_bytes))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl["seed"])
    W = [torch.empty((sp["b"], sp["a"]), dtype=torch.float16, device="cuda").normal_(
        0.0, sp["a"] ** -0.5, generator=gen) for sp in wl["layers"][:per * nb]]
    x = torch.randn((M, wl["layers"][0]["a"]), dtype=torch.float16, device="cuda", generator=gen)
    kap = lb_synth.kappa(2 if wl["layers"][0]["residual"] else 1)

    def fwd():
        h, li = x, 0
        for _ in range(nb):
            for n in ub:
                acc = F.linear(h, W[li])
                for k in range(1, n):
                    acc = acc + F.linear(h, W[li + k])
                li += n
                h = acc * (kap / math.sqrt(n))
        return h

    ms = _time_eager(torch, fwd, reps)
    del W
    torch.cuda.empty_cache()
    per_block = ms / nb
    ours_block = ours_ms / wl["blocks"]
    return {"what": "same wiring, dense fp16 weights, torch.nn.functional.linear; random weights, timing only",
            "blocks_timed": nb, "us_per_block": round(per_block * 1e3, 2),
            "weight_GBs": round(blk_bytes / (per_block * 1e-3) / 1e9, 1),
            "littlebit_us_per_block": round(ours_block * 1e3, 3),
            "speedup_of_littlebit": round(per_block / ours_block, 2)}


def factored_library_reference(torch, wl: dict, M: int, ours_ms: float, reps: int = 5) -> dict:
    """The LittleBit contractions of the matrix-core path with their operands
    materialised in fp16 and run through torch.matmul (the platform's GEMM
    library): per unit T = x . B1 (the unit's +-g l columns side by side),
    per layer y = T[:, its columns] . B2 (its +-h rows of both paths stacked),
    the unit's outputs summed and scaled into the next input.  Random operands,
    timing only.  Context for the bit-expanding kernels, not a target."""
    ub = wl["units"][:len(wl["units"]) // wl["blocks"]]
    P = 2 if wl["layers"][0]["residual"] else 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl["seed"])

    def rnd(r, c):
        return torch.empty((r, c), dtype=torch.float16, device="cuda").normal_(0.0, r ** -0.5, generator=gen)

    ops, li = [], 0
    for _ in range(wl["blocks"]):
        for n in ub:
            lay = wl["layers"][li:li + n]
            li += n
            ks = [P * sp["s"] for sp in lay]
            ops.append((rnd(lay[0]["a"], sum(ks)), [rnd(k, sp["b"]) for k, sp in zip(ks, lay)], ks))
    x = torch.randn((M, wl["layers"][0]["a"]), dtype=torch.float16, device="cuda", generator=gen)
    kap = lb_synth.kappa(P)

    def fwd():
        h = x
        for B1, B2, ks in ops:
            T = torch.matmul(h, B1)
            c0, acc = 0, None
            for B, k in zip(B2, ks):
                y = torch.matmul(T[:, c0:c0 + k], B)
                acc = y if acc is None else acc + y
                c0 += k
            h = acc * (kap / math.sqrt(len(ks)))
        return h

    ms = _time_eager(torch, fwd, reps)
    del ops
    torch.cuda.empty_cache()
    return {"what": "same contractions, operands materialised in fp16, torch.matmul; random operands, timing only",
            "ms_per_step": round(ms, 4), "littlebit_ms_per_step": round(ours_ms, 4),
            "speedup_of_littlebit": round(ms / ours_ms, 2)}


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


def _blas_setup():
    """Every host core this process may use, with the BLAS thread count set to
    match; returns (cores, BLAS description, limiter context or None)."""
    cores = len(os.sched_getaffinity(0))
    name, ctx = "unknown", None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            name = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info)
        ctx = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        pass
    return cores, name, ctx


def cpu_baseline(wl: dict, M: int, budget_s: float) -> dict:
    """Time the float64 oracle on a bounded sample of the workload's layers."""
    import oracle
    cores, blas, ctx = _blas_setup()
    x = lb_synth.activations(M, wl["layers"][0]["a"], seed=wl["seed"])
    done_bytes, done_layers, t_used = 0, 0, 0.0
    one = {"layers": None}
    try:
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
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "blas": blas,
            "sample": f"first {done_layers} of {len(wl['layers'])} matrices, M={M}, "
                      f"float64 numpy incl. bit unpack, {t_used:.1f} s, BLAS threads = cores"}


def validate(torch, stack, x, y, M, mode):
    """The timed output must be a valid sweep: no device-side wait gave up
    (lb_stack_check), and a traced run of the same input (every layer's
    output stored on the way) gives the same y, bit for bit where both runs
    take the same kernels (M = 1 sweep, M >= 64 unit kernels, or mode 1),
    else within the parity bar of the two runs.  Raises on failure."""
    stack.check()
    y_timed = y.clone()
    trace = torch.empty(stack.trace_elems(M), dtype=torch.float16, device="cuda")
    y2 = torch.empty_like(y)
    stack.forward(x, y2, trace)
    torch.cuda.synchronize()
    stack.check()
    same_kernels = M == 1 or M >= 64 or mode == 1
    if torch.equal(y_timed.view(torch.int16), y2.view(torch.int16)):
        return "timed y == traced run, bit for bit; lb_stack_check ok"
    if same_kernels:
        raise SystemExit("bench: the timed output differs from a traced run of the same input")
    if M <= 8:
        # a few rows may run as one batch-1 sweep per row: then each row
        # equals its own traced batch-1 sweep bit for bit
        t1 = torch.empty(stack.trace_elems(1), dtype=torch.float16, device="cuda")
        rows_equal = True
        for m in range(M):
            ym = torch.empty_like(y[m:m + 1])
            stack.forward(x[m:m + 1], ym, t1)
            torch.cuda.synchronize()
            rows_equal = rows_equal and torch.equal(ym.view(torch.int16), y_timed[m:m + 1].view(torch.int16))
        stack.check()
        if rows_equal:
            return "timed y == traced batch-1 sweep of every row, bit for bit; lb_stack_check ok"
    # other kernels than the traced run: two valid paths through a whole
    # stack (each layer within the parity bar) drift apart over the chain
    a, b = y_timed.double(), y2.double()
    rel = float((a - b).norm() / b.norm().clamp_min(1e-300))
    if not (torch.isfinite(a).all() and rel <= 1e-2):
        raise SystemExit(f"bench: the timed output differs from a traced run (rel L2 {rel:.2e})")
    return f"timed y vs traced run (other kernels): rel L2 {rel:.1e}; lb_stack_check ok"


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
    ap.add_argument("--timeline", action="store_true",
                    help="also record one batch-1 sweep's per-phase device timestamps (timeline object)")
    ap.add_argument("--no-fp16-reference", action="store_true",
                    help="skip the dense fp16 / library references (torch on random weights)")
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
        checked = validate(torch, stack, x, y, M, args.mode)
        print(f"[bench] {name}: {checked}", file=sys.stderr, flush=True)
        nbytes, flops = algorithmic_bytes(wl, M), algorithmic_flops(wl, M)
        res = {"wl": wl, "M": M, "ms": ms, "wall_ms": wall_ms, "bytes": nbytes, "flops": flops,
               "validated": checked}
        if len(wl["layers"]) == 1:
            # a single matrix: also the latency of one lb_forward call on it
            L0 = stack.layers[0]
            for _ in range(20):
                L0.forward(x, y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(200):
                L0.forward(x, y)
            e1.record()
            torch.cuda.synchronize()
            res["layer_forward_us_eager"] = round(e0.elapsed_time(e1) / 200 * 1e3, 3)
            # device time per call: 100 calls captured in a graph, replayed
            # (the eager figure can be bound by the host's launch rate)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(100):
                    L0.forward(x, y)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res["layer_forward_us"] = round(e0.elapsed_time(e1) / 1000 * 1e3, 3)
            del g
        if args.timeline and M == 1 and args.mode != 1:
            print("[bench] one sweep with device timestamps", file=sys.stderr, flush=True)
            res["timeline"] = sweep_timeline(torch, lbm, stack, x, y, len(wl["units"]))
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
        "validated": r["validated"],
        **({"layer_forward_us": r["layer_forward_us"],
            "layer_forward_us_eager": r["layer_forward_us_eager"]} if "layer_forward_us" in r else {}),
        "roofline": {"bound": "hbm" if batch1 else "mfma",
                     "achieved": round(gbs if batch1 else tflops, 3),
                     "peak": HBM_PEAK_GBS if batch1 else MFMA_FP16_PEAK_TFLOPS,
                     "unit": "GB/s" if batch1 else "TFLOP/s",
                     "frac": round((gbs / HBM_PEAK_GBS) if batch1 else (tflops / MFMA_FP16_PEAK_TFLOPS), 4),
                     "traffic": traffic,
                     "kernel": kernel_desc(M, args.mode)},
    }
    if "cpu" in r:
        out["cpu_baseline"] = r["cpu"]
    if "timeline" in r:
        out["timeline"] = r["timeline"]
    if not args.no_fp16_reference:
        print("[bench] timing the dense fp16 reference", file=sys.stderr, flush=True)
        out["dense_fp16_reference"] = dense_fp16_reference(torch, wl, M, ms)
    if batch1 and r["bytes"] <= MALL_BYTES // 2:
        # a working set that fits the MALL: also set against a measured MALL read rate
        ref = mall_reference(torch, r["bytes"])
        ref["stack_frac_of_mall_read"] = round(gbs / ref["read_GBs"], 4)
        out["mall_reference"] = ref
    if args.secondary and args.secondary != args.workload:
        s2 = measure(args.secondary, None, False)
        ms2 = s2["ms"]
        out["secondary"] = {"workload": args.secondary, "M": s2["M"], "ms_per_step": round(ms2, 5),
                            "us_per_layer": round(ms2 * 1e3 / s2["wl"]["blocks"], 3),
                            "TFLOP/s": round(s2["flops"] / (ms2 * 1e-3) / 1e12, 3),
                            "mfma_frac": round(s2["flops"] / (ms2 * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                            "GB/s": round(s2["bytes"] / (ms2 * 1e-3) / 1e9, 2),
                            "tokens_per_s_equiv": round(s2["M"] / (ms2 * 1e-3), 1),
                            "kernel": kernel_desc(s2["M"], args.mode),
                            "validated": s2["validated"]}
        if not args.no_fp16_reference:
            print("[bench] timing the fp16 references of the secondary workload", file=sys.stderr, flush=True)
            out["secondary"]["dense_fp16_reference"] = dense_fp16_reference(torch, s2["wl"], s2["M"], ms2)
            out["secondary"]["factored_library_reference"] = factored_library_reference(
                torch, s2["wl"], s2["M"], ms2)
    if not args.no_init:
        print("[bench] timing initialisation from real factors", file=sys.stderr, flush=True)
        out["init"] = measure_init(torch, lbm, with_cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
