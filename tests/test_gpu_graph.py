"""Forward calls captured into a HIP graph (torch.cuda.CUDAGraph: the
library launches on the current stream, which inside the capture is the
capture stream) and replayed.

Every replay runs after ordinary eager work has written a new input into
the captured buffer, and must equal the eager result for that input bit for
bit.  This covers the wave path, the matrix-core path, the one-launch sweep
(whose exchange generation lives in device memory, so replays of one
captured launch stay distinct), the sweep run once per row (M = 2: two
captured launches in a row), and stacks at M = 3, 8 and 128 (one launch).
"""
import numpy as np
import pytest

import lb_synth
from tests import lbtest
from tests.lbtest import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbm():
    lbtest.torch_dev()
    return lbtest.ensure_built()


def _replays_match_eager(torch, run, x, y, inputs):
    refs = []
    for xin in inputs:
        x.copy_(xin)
        run()
        torch.cuda.synchronize()
        refs.append(y.clone())
    g = torch.cuda.CUDAGraph()
    x.copy_(inputs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for k, xin in enumerate(inputs):
        x.copy_(xin)      # eager work between replays
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, refs[k]), f"replay {k} differs from the eager result"
        assert torch.isfinite(y.float()).all()


def _inputs(torch, M, a, n=3):
    return [torch.from_numpy(lb_synth.activations(M, a, seed=100 + k)).cuda() for k in range(n)]


@pytest.mark.parametrize("M", [1, 7, 70])
def test_layer_forward_in_a_graph(lbm, M):
    torch = lbtest.torch_dev()
    a, b, s = 1000, 600, 40
    say(f"[case] graph layer M={M}")
    L = lbm.Layer.from_paths(lb_synth.layer_inputs(a, b, s, True, seed=3))
    x = torch.empty((M, a), dtype=torch.float16, device="cuda")
    y = torch.empty((M, b), dtype=torch.float16, device="cuda")
    _replays_match_eager(torch, lambda: L.forward(x, y), x, y, _inputs(torch, M, a))


@pytest.mark.parametrize("name,blocks,M", [("llama7b_mlp_stack", 2, 1), ("llama7b_mlp_stack", 2, 2),
                                           ("llama7b_mlp_stack", 2, 3), ("llama7b_mlp_stack", 2, 8),
                                           ("llama7b_full_stack_M128", 1, 128)])
def test_stack_forward_in_a_graph(lbm, name, blocks, M):
    torch = lbtest.torch_dev()
    say(f"[case] graph stack {name} blocks={blocks} M={M}")
    wl = lb_synth.workload(name, blocks)
    layers = [lbm.Layer.from_paths(lb_synth.workload_layer_inputs(sp)) for sp in wl["layers"]]
    S = lbm.Stack(layers, wl["units"], lb_synth.kappa(2))
    S.reserve(M)
    a0, bl = wl["layers"][0]["a"], wl["layers"][-1]["b"]
    x = torch.empty((M, a0), dtype=torch.float16, device="cuda")
    y = torch.empty((M, bl), dtype=torch.float16, device="cuda")
    _replays_match_eager(torch, lambda: S.forward(x, y), x, y, _inputs(torch, M, a0))
    S.check()
