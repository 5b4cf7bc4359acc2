"""GPU parity of stacks (chained layers) through the C ABI.

Parity is teacher-forced per layer: each layer's fp16 output in the trace
is compared with the float64 oracle applied to the fp16 input the GPU
actually fed it, so errors do not compound along the chain.  Each unit
input is checked against the combine of the previous unit's fp16 outputs
(fp16 of kappa/sqrt(n) * sum, computed in float64) to within one fp16 ulp.
"""
import math

import numpy as np
import pytest

import lb_synth
import oracle
from tests import lbtest
from tests.lbtest import assert_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbm():
    lbtest.torch_dev()
    return lbtest.ensure_built()


def build_stack(lbm, name, blocks=None, keep_paths=True):
    wl = lb_synth.workload(name, blocks)
    layers, paths = [], []
    for spec in wl["layers"]:
        p = lb_synth.workload_layer_inputs(spec)
        layers.append(lbm.Layer.from_paths(p))
        paths.append(p if keep_paths else None)
    P = 2 if wl["layers"][0]["residual"] else 1
    S = lbm.Stack(layers, wl["units"], lb_synth.kappa(P))
    return wl, S, paths


def run_stack(lbm, wl, S, M, mode=0):
    torch = lbtest.torch_dev()
    a0 = wl["layers"][0]["a"]
    b_last = wl["layers"][-1]["b"]
    x0 = lb_synth.activations(M, a0, seed=wl["seed"])
    xd = lbtest.to_dev(x0)
    y = torch.empty((M, b_last), dtype=torch.float16, device="cuda")
    tr = torch.empty(S.trace_elems(M), dtype=torch.float16, device="cuda")
    S.set_mode(mode)
    S.forward(xd, y, tr)
    torch.cuda.synchronize()
    return x0, y.cpu().numpy(), tr.cpu().numpy()


def split_trace(wl, tr, M):
    Ys, Xs, off = [], [], 0
    for spec in wl["layers"]:
        Ys.append(tr[off:off + M * spec["b"]].reshape(M, spec["b"]))
        off += M * spec["b"]
    ub = np.cumsum([0] + wl["units"][:-1])
    for u, b0 in enumerate(ub):
        a = wl["layers"][b0]["a"]
        Xs.append(tr[off:off + M * a].reshape(M, a))
        off += M * a
    assert off == tr.size
    return Ys, Xs, ub


def check_combine(got, ys, c):
    """got == fp16(c * sum ys) within one fp16 ulp (float64 reference)."""
    ref = oracle.combine(ys, c).astype(np.float64)
    g = got.astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert (np.abs(g - ref) <= ulp).all(), float(np.max(np.abs(g - ref) / ulp))


def check_stack(wl, paths, x0, y, tr, M, sample=None):
    Ys, Xs, ub = split_trace(wl, tr, M)
    kap = lb_synth.kappa(2 if wl["layers"][0]["residual"] else 1)
    assert np.array_equal(Xs[0], x0)
    units = wl["units"]
    idx = list(range(len(wl["layers"]))) if sample is None else sample
    unit_of = np.repeat(np.arange(len(units)), units)
    for li in idx:
        u = unit_of[li]
        say(f"[check] layer {li} (unit {u})")
        p = paths[li] if paths[li] is not None else lb_synth.workload_layer_inputs(wl["layers"][li])
        assert_parity(Ys[li], oracle.forward(Xs[u], p), f"layer {li}")
    for u in range(1, len(units)):
        prev = list(range(ub[u - 1], ub[u - 1] + units[u - 1]))
        check_combine(Xs[u], [Ys[i] for i in prev], kap / math.sqrt(units[u - 1]))
    last = list(range(ub[-1], ub[-1] + units[-1]))
    check_combine(y, [Ys[i] for i in last], kap / math.sqrt(units[-1]))


@pytest.mark.parametrize("M", [1, 3])
def test_mlp_stack_two_blocks(lbm, M):
    wl, S, paths = build_stack(lbm, "llama7b_mlp_stack", blocks=2)
    say(f"[case] mlp stack 2 blocks M={M}")
    x0, y, tr = run_stack(lbm, wl, S, M)
    check_stack(wl, paths, x0, y, tr, M)


@pytest.mark.parametrize("mode", [0, 1])
def test_full_block_stack_M128(lbm, mode):
    """Mode 0 runs one unit (q/k/v, o, gate/up, down) per launch pair with
    the combine fused; mode 1 runs each layer alone, then a combine."""
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    say(f"[case] full block stack M=128 mode={mode}")
    x0, y, tr = run_stack(lbm, wl, S, 128, mode=mode)
    check_stack(wl, paths, x0, y, tr, 128)


@pytest.mark.parametrize("M", [64, 70, 257])
def test_unit_path_odd_widths(lbm, M):
    wl, S, paths = _odd_stack(lbm)
    say(f"[case] unit path odd widths M={M}")
    x0, y, tr = run_stack(lbm, wl, S, M, mode=0)
    check_stack(wl, paths, x0, y, tr, M)
    _, y1, _ = run_stack(lbm, wl, S, M, mode=1)
    assert_parity(y.astype(np.float64), y1.astype(np.float64), "unit vs per-layer")


@pytest.mark.parametrize("M", [64, 130])
def test_unit_path_single_path_wide_unit(lbm, M):
    """The matrix-core unit kernels on one-path layers: a four-layer unit
    (2000 latent columns) and an odd single layer."""
    shapes = [(3000, 1000, 500)] * 4 + [(1000, 3000, 37)]
    wl, S, paths = _odd_stack(lbm, seed=11, residual=False, shapes=shapes, units=[4, 1])
    say(f"[case] unit path single path, wide unit M={M}")
    x0, y, tr = run_stack(lbm, wl, S, M, mode=0)
    check_stack(wl, paths, x0, y, tr, M, sample=[0, 3, 4])
    _, y1, _ = run_stack(lbm, wl, S, M, mode=1)
    assert_parity(y.astype(np.float64), y1.astype(np.float64), "unit vs per-layer")


def test_unit_path_repeated_and_deterministic(lbm):
    """Split-K partial sums are combined in a fixed order: repeated batched
    runs are bitwise identical, and the tile counters are left at zero."""
    torch = lbtest.torch_dev()
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    say("[case] unit path repeated M=128")
    x0, y, tr = run_stack(lbm, wl, S, 128, mode=0)
    xd = lbtest.to_dev(x0)
    outs = []
    for _ in range(10):
        y2 = torch.empty((128, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
        S.forward(xd, y2, None)
        outs.append(y2)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint16), y.view(np.uint16))


def test_stack_without_trace_matches_trace_run(lbm):
    torch = lbtest.torch_dev()
    wl, S, paths = build_stack(lbm, "llama7b_mlp_stack", blocks=2)
    x0, y, tr = run_stack(lbm, wl, S, 1)
    xd = lbtest.to_dev(x0)
    y2 = torch.empty_like(torch.from_numpy(y)).cuda()
    S.forward(xd, y2, None)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), y.view(np.uint16))


def _odd_stack(lbm, seed=5, residual=True, shapes=None, units=None):
    """A small stack with widths that are not multiples of 16 (by default)."""
    if shapes is None:
        shapes = [(100, 37, 5), (100, 37, 5), (37, 70, 33), (70, 100, 17), (70, 100, 17)]
        units = [2, 1, 2]
    layers, paths = [], []
    for i, (a, b, s) in enumerate(shapes):
        p = lb_synth.layer_inputs(a, b, s, residual, seed=seed, layer=i)
        for q in p:
            q["a"], q["b"], q["s"] = a, b, s
        layers.append(lbm.Layer.from_paths(p))
        paths.append(p)
    wl = {"name": "odd", "seed": seed, "M": 1, "units": units,
          "layers": [{"a": a, "b": b, "s": s, "residual": residual} for (a, b, s) in shapes]}
    return wl, lbm.Stack(layers, units, lb_synth.kappa(2 if residual else 1)), paths


# The first product's column width (1, 2 or 4 per thread) is chosen per unit:
# the 70B MLP stack takes 2 (gate/up) and 1 (down), the 7B full block 4 (the
# attention units) and 2 (its MLP), tiny_256 1.
@pytest.mark.parametrize("name,blocks", [("llama7b_mlp_stack", 3), ("llama70b_mlp_stack", 2),
                                         ("llama7b_attn_proj_4096", 1), ("tiny_256", 1),
                                         ("llama7b_full_stack_M128", 2)])
def test_persistent_sweep_parity(lbm, name, blocks):
    wl, S, paths = build_stack(lbm, name, blocks=blocks)
    say(f"[case] persistent sweep {name} blocks={blocks}")
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    check_stack(wl, paths, x0, y, tr, 1)
    # the per-layer kernels reach the same result within the parity bar
    _, y1, _ = run_stack(lbm, wl, S, 1, mode=1)
    assert_parity(y.astype(np.float64), y1.astype(np.float64), "persistent vs per-layer")


def test_llama70b_full_length_sweep(lbm):
    """The measured configuration at full length: 80 blocks (240 matrices,
    161 phases) in one launch with the trace.  Layers 0, 119 and 239 against
    the oracle (teacher-forced) and every one of the 160 combines within one
    fp16 ulp; an untraced sweep of the same input gives the same y bit for
    bit, as bench.py's timed runs do."""
    torch = lbtest.torch_dev()
    say("[case] llama70b_mlp_stack, 80 blocks, one launch")
    wl, S, paths = build_stack(lbm, "llama70b_mlp_stack", keep_paths=False)
    assert len(wl["layers"]) == 240
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    check_stack(wl, paths, x0, y, tr, 1, sample=[0, 119, 239])
    xd = lbtest.to_dev(x0)
    y2 = torch.empty((1, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
    S.forward(xd, y2, None)
    torch.cuda.synchronize()
    S.check()
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), y.view(np.uint16))
    S.close()


def test_persistent_odd_widths(lbm):
    wl, S, paths = _odd_stack(lbm)
    say("[case] persistent odd widths")
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    check_stack(wl, paths, x0, y, tr, 1)


def test_persistent_single_path_wide_unit(lbm):
    """One path per layer: a unit of four 3000 -> 1000 layers with s = 500
    (2000 latent columns on one row tile per workgroup, so the first product
    takes four columns per thread), then an odd 1000 -> 3000 layer (s = 37,
    one column per thread)."""
    shapes = [(3000, 1000, 500)] * 4 + [(1000, 3000, 37)]
    wl, S, paths = _odd_stack(lbm, seed=11, residual=False, shapes=shapes, units=[4, 1])
    say("[case] persistent single path, wide unit")
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    check_stack(wl, paths, x0, y, tr, 1)


def test_persistent_repeated_and_deterministic(lbm):
    """Many launches in a row (generation counters advance) give bitwise
    identical outputs, with and without the trace."""
    torch = lbtest.torch_dev()
    wl, S, paths = build_stack(lbm, "llama7b_mlp_stack", blocks=4)
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    xd = lbtest.to_dev(x0)
    outs = []
    for _ in range(20):
        y2 = torch.empty((1, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
        S.forward(xd, y2, None)
        outs.append(y2)
    torch.cuda.synchronize()
    S.check()
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint16), y.view(np.uint16))


def test_persistent_wait_failure_is_reported_and_recovers(lbm):
    """Failure path of the one-launch sweep, forced from the host: every
    device-side wait waits for words nobody writes (short bound), so the
    kernel ends normally; the next lb_stack_forward reports LB_ETIMEOUT
    (and runs nothing), lb_stack_check reports it too, and the sweep after
    that resets the synchronisation words and is correct again."""
    torch = lbtest.torch_dev()
    say("[case] persistent sweep with unsatisfiable waits")
    wl, S, paths = build_stack(lbm, "llama7b_mlp_stack", blocks=2)
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    xd = lbtest.to_dev(x0)
    y2 = torch.empty((1, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
    lbm.lb_stack_test_wait_failure(S.handle, True)
    S.forward(xd, y2, None)
    torch.cuda.synchronize()
    lbm.lb_stack_test_wait_failure(S.handle, False)
    # the next forward after the failed sweep finished reports it, runs nothing
    with pytest.raises(lbm.LBError) as ei:
        S.forward(xd, y2, None)
    assert ei.value.status == lbm.LB_ETIMEOUT
    with pytest.raises(lbm.LBError) as ei:
        S.check()
    assert ei.value.status == lbm.LB_ETIMEOUT
    for _ in range(3):
        S.forward(xd, y2, None)
    torch.cuda.synchronize()
    S.check()
    assert np.array_equal(y2.cpu().numpy().view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("name,blocks", [("llama7b_mlp_stack", 3), ("llama70b_mlp_stack", 2)])
def test_persistent_sweep_under_random_delays(lbm, name, blocks):
    """Exchange stress: with the host-selected delay mode every wave of the
    one-launch sweep waits a pseudo-random time before each exchange step
    (publish, intra-XCD sum, cross-XCD store and poll, final poll), so the
    workgroups meet in orders an undisturbed sweep never produces.  Every
    delayed sweep, traced or not, must equal the undelayed one bit for bit
    (fixed summation order), and no wait may give up."""
    torch = lbtest.torch_dev()
    say(f"[case] delayed sweeps {name} blocks={blocks}")
    wl, S, paths = build_stack(lbm, name, blocks=blocks)
    x0, y, tr = run_stack(lbm, wl, S, 1, mode=2)
    S.check()
    n = len(wl["layers"])
    check_stack(wl, paths, x0, y, tr, 1, sample=[0, n - 1])
    xd = lbtest.to_dev(x0)
    yd = torch.empty((1, wl["layers"][-1]["b"]), dtype=torch.float16, device="cuda")
    td = torch.empty(tr.size, dtype=torch.float16, device="cuda")
    for seed, ticks in [(1, 200), (2, 2000), (3, 20000)]:
        say(f"[case] delays seed={seed} up to {ticks} ticks")
        lbm.lb_stack_test_delay(S.handle, seed, ticks)
        for rep in range(3):
            yd.zero_()
            S.forward(xd, yd, None)
            torch.cuda.synchronize()
            S.check()
            assert np.array_equal(yd.cpu().numpy().view(np.uint16), y.view(np.uint16)), (seed, rep)
        td.zero_()
        S.forward(xd, yd, td)
        torch.cuda.synchronize()
        S.check()
        assert np.array_equal(td.cpu().numpy().view(np.uint16), tr.view(np.uint16)), f"trace, seed {seed}"
    lbm.lb_stack_test_delay(S.handle, 0, 0)
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_stack_test_delay(S.handle, 1, 100001)
    assert ei.value.status == lbm.LB_EINVAL


@pytest.mark.parametrize("name,M", [("llama7b_mlp_stack", 2), ("llama70b_mlp_stack", 2)])
def test_small_batch_without_trace_runs_rows_as_batch1(lbm, name, M):
    """For M = 2 without a trace the automatic mode runs the batch-1 sweep
    once per row (from 3 rows the one-launch stack): every row
    equals its own M = 1 result bit for bit (the M = 1 sweep is checked
    against the oracle above), and the batch agrees at the parity bar with
    the per-layer kernels that the same M uses when a trace is asked for."""
    torch = lbtest.torch_dev()
    say(f"[case] small batch without trace {name} M={M}")
    wl, S, paths = build_stack(lbm, name, blocks=2)
    x0, yt, tr = run_stack(lbm, wl, S, M)
    check_stack(wl, paths, x0, yt, tr, M, sample=[0, 2, 5])
    b_last = wl["layers"][-1]["b"]
    xd = lbtest.to_dev(x0)
    y = torch.empty((M, b_last), dtype=torch.float16, device="cuda")
    S.forward(xd, y, None)
    rows = []
    for m in range(M):
        ym = torch.empty((1, b_last), dtype=torch.float16, device="cuda")
        S.forward(xd[m:m + 1].contiguous(), ym, None)
        rows.append(ym)
    torch.cuda.synchronize()
    S.check()
    got = y.cpu().numpy()
    for m in range(M):
        assert np.array_equal(got[m:m + 1].view(np.uint16), rows[m].cpu().numpy().view(np.uint16))
    assert_parity(got, yt.astype(np.float64), f"per-row sweeps vs per-layer kernels M={M}")
