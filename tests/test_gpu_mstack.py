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


def test_one_launch_rows_follow_the_oracle_chain(lbm):
    """Untraced one-launch output on sampled rows against the oracle's own
    chain: every layer and combine computed in float64 from the previous
    unit's fp16-rounded combine (the rounding the stack performs)."""
    torch = lbtest.torch_dev()
    say("[case] one-launch M=70 vs the oracle chain")
    wl, S, paths = build_stack(lbm, "llama7b_full_stack_M128", blocks=1)
    M = 70
    x0 = lb_synth.activations(M, wl["layers"][0]["a"], seed=wl["seed"])
    y = _untraced(torch, S, lbtest.to_dev(x0), wl["layers"][-1]["b"], M, 3)
    kap = lb_synth.kappa(2)
    rows = [0, 33, 69]
    x = x0[rows].astype(np.float64)
    b0 = 0
    for nu in wl["units"]:
        ys = [oracle.forward(x.astype(np.float16), paths[b0 + k]).astype(np.float16) for k in range(nu)]
        x = (kap / math.sqrt(nu)) * np.sum([v.astype(np.float64) for v in ys], axis=0)
        b0 += nu
    assert_parity(y[rows], x, "one-launch stack vs oracle chain")
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
