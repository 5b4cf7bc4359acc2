"""lb_forward_noalloc: the layer forward with its scratch in the library's
fixed device array (for callers that cannot allocate), through the C ABI.

For M >= 2 it runs the same kernels as lb_forward, so on the same input
its output is the same bit for bit; for one row of a small layer (a <=
4096, P s <= 256) lb_forward takes its one-launch kernel (different chunking of the first product) while this
entry point keeps the three-launch wave path, so the two agree at the
parity bar.  Both always meet the oracle's bar (layer definition: Samsung
LittleBit news page, aifrontier.co.jp, Sec. 2).  Each case makes
two calls in a row, the second with a smaller input (the array keeps the
first call's contents).
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


def _both(lbm, torch, L, paths, xh, what):
    M, b = xh.shape[0], paths[0]["b"]
    x = lbtest.to_dev(xh)
    y_ref = torch.empty((M, b), dtype=torch.float16, device="cuda")
    y_na = torch.full((M, b), float("nan"), dtype=torch.float16, device="cuda")
    lbm.lb_forward(L.handle, x, y_ref, M)
    lbm.lb_forward_noalloc(L.handle, x, y_na, M)
    torch.cuda.synchronize()
    if M >= 2:
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), f"{what}: differs from lb_forward"
    else:
        assert_parity(y_na.cpu().numpy().astype(np.float64), y_ref.cpu().numpy().astype(np.float64),
                      f"{what} vs lb_forward")
    ref = oracle.forward(xh, paths)
    assert_parity(y_na.cpu().numpy(), ref, what)
    assert_parity(y_ref.cpu().numpy(), ref, f"{what} (lb_forward)")


@pytest.mark.parametrize("a,b,s,res,Ms", [(4096, 11008, 133, True, (70, 5)),
                                          (1000, 600, 40, True, (130, 1)),
                                          (11008, 4096, 133, True, (63, 2)),
                                          (257, 129, 63, False, (64, 3))])
def test_noalloc_matches_lb_forward(lbm, a, b, s, res, Ms):
    torch = lbtest.torch_dev()
    paths = lb_synth.layer_inputs(a, b, s, res, seed=a + s)
    L = lbm.Layer.from_paths(paths)
    for k, M in enumerate(Ms):
        say(f"[case] noalloc a={a} b={b} s={s} call {k} M={M}")
        _both(lbm, torch, L, paths, lb_synth.activations(M, a, seed=M + k), f"noalloc M={M}")
    L.close()


def test_noalloc_rejects_what_does_not_fit(lbm):
    """A layer whose matrix-core scratch exceeds the array: LB_EUNSUPPORTED
    at M >= 64 with nothing launched; its wave path still fits and runs."""
    torch = lbtest.torch_dev()
    a, b, s = 64, 64, 4096
    paths = lb_synth.layer_inputs(a, b, s, True, seed=9)
    L = lbm.Layer.from_paths(paths)
    say("[case] noalloc too large for the matrix-core path")
    x = lbtest.to_dev(lb_synth.activations(64, a, seed=1))
    y = torch.zeros((64, b), dtype=torch.float16, device="cuda")
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_forward_noalloc(L.handle, x, y, 64)
    assert ei.value.status == lbm.LB_EUNSUPPORTED
    assert "scratch" in lbm.lb_last_error()
    torch.cuda.synchronize()
    assert not y.any()
    say("[case] noalloc wave path of the same layer")
    _both(lbm, torch, L, paths, lb_synth.activations(3, a, seed=2), "noalloc wave path, s = 4096")
    L.close()


def test_noalloc_needs_the_matrix_core_copy_built(lbm):
    """At M >= 64 the entry point allocates nothing, so on a layer whose
    matrix-core sign copy is not built yet it returns LB_ENOTREADY with
    nothing launched; after lb_prepare it matches lb_forward bit for bit."""
    torch = lbtest.torch_dev()
    a, b, s = 1000, 600, 40
    paths = lb_synth.layer_inputs(a, b, s, True, seed=31)
    L = lbm.Layer.from_paths(paths)
    say("[case] noalloc M=80 before lb_prepare")
    x = lbtest.to_dev(lb_synth.activations(80, a, seed=3))
    y = torch.zeros((80, b), dtype=torch.float16, device="cuda")
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_forward_noalloc(L.handle, x, y, 80)
    assert ei.value.status == lbm.LB_ENOTREADY
    assert "lb_prepare" in lbm.lb_last_error()
    torch.cuda.synchronize()
    assert not y.any()
    L.prepare(80)
    say("[case] noalloc M=80, 65 after lb_prepare")
    for k, M in enumerate((80, 65)):
        _both(lbm, torch, L, paths, lb_synth.activations(M, a, seed=10 + k), f"noalloc prepared M={M}")
    L.close()
