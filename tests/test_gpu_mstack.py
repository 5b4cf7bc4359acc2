"""The one-launch M >= 64 stack (include/lb.h, lb_stack_set_mode 3): every
unit's matrix-core tiles as work items of one launch, pipelined by 32-row
block (mode 3, and the automatic mode without a trace, from M = 64).  It
runs the same tiles, with the same splits and summation order, as the two
launches per unit (which a traced call runs), so its output must equal
theirs bit for bit; the traced call's layers and combines
are checked against the float64 oracle (layer definition: [LB news]
Sec. 2), and the untraced result against the oracle's chain on sampled
rows."""
import math

import numpy as np
import pytest

import lb_synth
import oracle
from tests import lbtest
from tests.lbtest import assert_parity, say
from tests.test_gpu_stack import build_stack, check_stack, run_stack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbm():
    lbtest.torch_dev()
    return lbtest.ensure_built()


def _oracle_chain(wl, paths, x0, rows):
    """The oracle's own chain on the given rows: every layer and combine in
    float64 from the previous unit's fp16-rounded combine (the rounding the
    stack performs); residual layers (kappa for two paths)."""
    kap = lb_synth.kappa(2)
    x = x0[rows].astype(np.float64)
    b0 = 0
    for nu in wl["units"]:
        ys = [oracle.forward(x.astype(np.float16), paths[b0 + k]).astype(np.float16) for k in range(nu)]
        x = (kap / math.sqrt(nu)) * np.sum([v.astype(np.float64) for v in ys], axis=0)
        b0 += nu
    return x


def _untraced(torch, S, xd, b_last, M, mode):
    y = torch.full((M, b_last), float("nan"), dtype=torch.float16, device="cuda")
    S.set_mode(mode)
    S.forward(xd, y, None)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name,blocks,M", [("llama7b_full_stack_M128", 2, 128),
                                           ("llama7b_full_stack_M128", 1, 64),
                                           ("llama7b_full_stack_M128", 1, 100),
                                           ("llama7b_full_stack_M128", 1, 256),
                                           ("llama7b_full_stack_M128", 1, 300),
                                           ("llama7b_mlp_stack", 3, 96)])
def test_one_launch_equals_unit_launches(lbm, name, blocks, M):
    torch = lbtest.torch_dev()
    say(f"[case] one-launch M>=64 stack {name} blocks={blocks} M={M}")
    wl, S, paths = build_stack(lbm, name, blocks=blocks)
    x0, yt, tr = run_stack(lbm, wl, S, M)  # traced: two launches per unit
    n = len(wl["layers"])
    check_stack(wl, paths, x0, yt, tr, M, sample=[0, n // 2, n - 1])
    xd = lbtest.to_dev(x0)
    b_last = wl["layers"][-1]["b"]
    y0 = _untraced(torch, S, xd, b_last, M, 0)
    assert np.array_equal(y0.view(np.uint16), yt.view(np.uint16)), "automatic mode: untraced != traced"
    for rep in range(3):
        y3 = _untraced(torch, S, xd, b_last, M, 3)
        S.check()
        assert np.array_equal(y3.view(np.uint16), yt.view(np.uint16)), f"one launch differs (call {rep})"
    S.close()


@pytest.mark.parametrize("M", [5, 70])
def test_one_launch_rows_follow_the_oracle_chain(lbm, M):
    """Untraced one-launch output on sampled rows against the oracle's own
    chain: every layer and combine computed in float64 from the previous
    unit's fp16-rounded combine (the rounding the stack performs)."""
    torch = lbtest.torch_dev()
    say(f"[case] one-launch M={M} vs the oracle chain")
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    x0 = lb_synth.activations(M, wl["layers"][0]["a"], seed=wl["seed"])
    y = _untraced(torch, S, lbtest.to_dev(x0), wl["layers"][-1]["b"], M, 3)
    rows = sorted({0, M // 2, M - 1})
    assert_parity(y[rows], _oracle_chain(wl, paths, x0, rows), "one-launch stack vs oracle chain")
    S.close()


def test_one_launch_graph_replays(lbm):
    """Captured after one eager call at the same M: every replay equals the
    eager result."""
    torch = lbtest.torch_dev()
    say("[case] one-launch M=128 in a graph")
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    M = 128
    x0 = lb_synth.activations(M, wl["layers"][0]["a"], seed=5)
    xd = lbtest.to_dev(x0)
    b_last = wl["layers"][-1]["b"]
    y = torch.empty((M, b_last), dtype=torch.float16, device="cuda")
    S.set_mode(3)
    S.forward(xd, y, None)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.forward(xd, y, None)
    torch.cuda.synchronize()
    for k in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {k}"
    S.check()
    S.close()


def test_automatic_mode_capture_before_setup_runs_unit_launches(lbm):
    """Automatic mode from M = 64 takes the one-launch stack, whose launch
    arguments are set up on the first eager call for a row count.  Captured
    before that, the call runs the two launches per unit instead; both
    graphs and the eager call must give the same output bit for bit (the
    same tiles in the same order)."""
    torch = lbtest.torch_dev()
    say("[case] automatic M=128: capture before and after the one-launch setup")
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    M = 128
    S.reserve(M)  # scratch and matrix-core sign copies, so the capture allocates nothing
    xd = lbtest.to_dev(lb_synth.activations(M, wl["layers"][0]["a"], seed=6))
    b_last = wl["layers"][-1]["b"]
    y = torch.empty((M, b_last), dtype=torch.float16, device="cuda")

    def captured():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            S.forward(xd, y, None)
        torch.cuda.synchronize()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return y.clone()

    y_units = captured()                  # not set up yet: two launches per unit
    S.forward(xd, y, None)                # eager: sets up and runs the one launch
    torch.cuda.synchronize()
    y_eager = y.clone()
    y_one = captured()                    # set up: the one launch
    S.check()
    assert torch.isfinite(y_eager.float()).all()
    assert torch.equal(y_units, y_eager), "captured unit launches differ from the eager one-launch call"
    assert torch.equal(y_one, y_eager), "captured one-launch call differs from the eager call"
    S.close()


@pytest.mark.parametrize("name,blocks,M", [("llama7b_mlp_stack", 3, 3), ("llama7b_mlp_stack", 2, 16),
                                           ("llama70b_mlp_stack", 2, 3), ("llama7b_full_stack_M128", 1, 40)])
def test_small_batch_runs_one_launch(lbm, name, blocks, M):
    """From 3 rows without a trace the automatic mode runs the one-launch
    stack: its output equals mode 3's bit for bit, repeated calls agree,
    and sampled rows meet the parity bar against the oracle's own chain.
    The traced call runs the wave-path kernels of each layer instead, each
    layer and combine checked against the oracle (teacher-forced)."""
    torch = lbtest.torch_dev()
    say(f"[case] small batch one launch {name} blocks={blocks} M={M}")
    wl, S, paths = build_stack(lbm, name, blocks=blocks)
    x0, yt, tr = run_stack(lbm, wl, S, M)  # traced: the wave path
    n = len(wl["layers"])
    check_stack(wl, paths, x0, yt, tr, M, sample=[0, n // 2, n - 1])
    xd = lbtest.to_dev(x0)
    b_last = wl["layers"][-1]["b"]
    y0 = _untraced(torch, S, xd, b_last, M, 0)
    S.check()
    y3 = _untraced(torch, S, xd, b_last, M, 3)
    y0b = _untraced(torch, S, xd, b_last, M, 0)
    S.check()
    assert np.array_equal(y0.view(np.uint16), y3.view(np.uint16)), "automatic mode != mode 3"
    assert np.array_equal(y0.view(np.uint16), y0b.view(np.uint16)), "repeated calls differ"
    rows = sorted({0, M // 2, M - 1})
    assert_parity(y0[rows], _oracle_chain(wl, paths, x0, rows), f"one launch vs oracle chain M={M}")
    S.close()


def test_small_batch_capture_before_setup_runs_wave_path(lbm):
    """Captured before the one launch is set up for its row count, an M = 8
    stack call runs the wave-path kernels instead (nothing is allocated
    under capture).  Its replays and the later eager one-launch call each
    meet the parity bar against the oracle's chain on sampled rows, and they
    are different kernels (fp16 latent on the matrix cores, fp32 in the
    wave path), so the replay differs from the eager output."""
    torch = lbtest.torch_dev()
    say("[case] automatic M=8: capture before the one-launch setup")
    wl, S, paths = build_stack(lbm, "llama7b_mlp_stack", blocks=2)
    M = 8
    S.reserve(M)  # scratch and matrix-core sign copies; the launch setup is per row count
    x0 = lb_synth.activations(M, wl["layers"][0]["a"], seed=8)
    xd = lbtest.to_dev(x0)
    b_last = wl["layers"][-1]["b"]
    y = torch.empty((M, b_last), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.forward(xd, y, None)
    torch.cuda.synchronize()
    y.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    y_wave = y.cpu().numpy()
    y_one = _untraced(torch, S, xd, b_last, M, 0)
    S.check()
    rows = [0, 3, 7]
    ref = _oracle_chain(wl, paths, x0, rows)
    assert_parity(y_wave[rows], ref, "captured wave path vs oracle chain")
    assert_parity(y_one[rows], ref, "eager one launch vs oracle chain")
    assert not np.array_equal(y_wave.view(np.uint16), y_one.view(np.uint16)), "the fallback did not run"
    S.close()
