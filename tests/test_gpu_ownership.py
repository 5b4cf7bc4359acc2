"""Workspace ownership of layers and stacks (include/lb.h conventions).

Every buffer a forward call writes belongs to the layer or stack it runs:
forward calls on different layers share nothing, a reservation never frees
memory an earlier launch may still use, and nothing is reallocated while
the object lives.  So a forward captured into a HIP graph stays valid after
other (larger) layers are created and run, and two layers can run on two
streams at once.  Every result is checked against the float64 oracle
(layer definition: Samsung LittleBit news page, aifrontier.co.jp, Sec. 2).
"""
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


@pytest.mark.parametrize("M", [1, 9, 70])
def test_captured_forward_survives_a_larger_layer(lbm, M):
    """Capture layer A's forward, create a much larger layer B and run it
    (its workspace is written), destroy it, then replay A: every replay is
    bit-identical to A's eager result and matches the oracle."""
    torch = lbtest.torch_dev()
    say(f"[case] capture, larger layer, replay M={M}")
    a, b, s = 700, 500, 37
    pa = lb_synth.layer_inputs(a, b, s, True, seed=41)
    A = lbm.Layer.from_paths(pa)
    xh = lb_synth.activations(M, a, seed=42)
    x = lbtest.to_dev(xh)
    y = torch.empty((M, b), dtype=torch.float16, device="cuda")
    A.forward(x, y)
    torch.cuda.synchronize()
    ref = y.clone()
    assert_parity(ref.cpu().numpy(), oracle.forward(xh, pa), "eager A")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.forward(x, y)
    torch.cuda.synchronize()
    for k in range(2):
        # a larger layer, created and run after the capture
        pb = lb_synth.layer_inputs(4096, 11008, 133, True, seed=43 + k)
        B = lbm.Layer.from_paths(pb)
        xb = lbtest.to_dev(lb_synth.activations(M, 4096, seed=44))
        yb = torch.empty((M, 11008), dtype=torch.float16, device="cuda")
        B.forward(xb, yb)
        torch.cuda.synchronize()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {k} after a larger layer differs"
        B.close()
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, ref), "replay after the larger layer was destroyed differs"
    A.close()


@pytest.mark.parametrize("M", [1, 5, 128])
def test_two_layers_on_two_streams(lbm, M):
    """Two layers run concurrently on two streams of default priority, many
    calls each without synchronising in between; each result matches the
    oracle and the last one of each stream equals a lone eager run."""
    torch = lbtest.torch_dev()
    say(f"[case] two layers, two streams, M={M}")
    specs = [(1024, 768, 61, 51), (768, 1024, 45, 52)]
    layers, paths, xs, ys, refs = [], [], [], [], []
    for a, b, s, seed in specs:
        p = lb_synth.layer_inputs(a, b, s, True, seed=seed)
        L = lbm.Layer.from_paths(p)
        xh = lb_synth.activations(M, a, seed=seed + 1)
        x = lbtest.to_dev(xh)
        y = torch.empty((M, b), dtype=torch.float16, device="cuda")
        L.forward(x, y)
        torch.cuda.synchronize()
        assert_parity(y.cpu().numpy(), oracle.forward(xh, p), f"lone layer {seed}")
        refs.append(y.clone())
        layers.append(L), paths.append(p), xs.append(x)
        ys.append([torch.empty((M, b), dtype=torch.float16, device="cuda") for _ in range(8)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i in range(8):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                layers[k].forward(xs[k], ys[k][i], stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        for i in range(8):
            assert torch.equal(ys[k][i], refs[k]), f"stream {k} call {i} differs from the lone run"
    for L in layers:
        L.close()


def test_stack_reserve_growth_keeps_captured_sweeps_valid(lbm):
    """A stack forward captured at M = 8 keeps replaying correctly after the
    stack's scratch grew to a larger reservation (the old scratch is retired,
    not freed, until the stack is destroyed)."""
    torch = lbtest.torch_dev()
    say("[case] stack reserve growth after capture")
    wl = lb_synth.workload("llama7b_mlp_stack", 1)
    layers = [lbm.Layer.from_paths(lb_synth.workload_layer_inputs(sp)) for sp in wl["layers"]]
    S = lbm.Stack(layers, wl["units"], lb_synth.kappa(2))
    M = 8
    a0, bl = wl["layers"][0]["a"], wl["layers"][-1]["b"]
    x = lbtest.to_dev(lb_synth.activations(M, a0, seed=61))
    y = torch.empty((M, bl), dtype=torch.float16, device="cuda")
    S.forward(x, y)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.forward(x, y)
    torch.cuda.synchronize()
    S.reserve(300)       # grows the scratch: the captured launches keep theirs
    x2 = lbtest.to_dev(lb_synth.activations(200, a0, seed=62))
    y2 = torch.empty((200, bl), dtype=torch.float16, device="cuda")
    S.forward(x2, y2)    # uses the new scratch
    torch.cuda.synchronize()
    for _ in range(2):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
    S.check()
    S.close()
