"""Device storage of a layer's signs (include/lb.h, lb_create / lb_prepare).

A layer holds its sign bits once, in the 16-row tile layouts that every
kernel for M < 64 reads, so its resident sign bytes match the bit count of
[LB2 column] Ch. 1 (s (a + b) bits per path) up to tile padding.  The
matrix-core copy is added by lb_prepare or by the first forward with
M >= 64; a forward of that kind under graph capture before it exists is
refused with LB_ENOTREADY instead of allocating.  Every result is checked
against the float64 oracle (layer definition: [LB news] Sec. 2).
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


def _fwd(torch, L, xh, b):
    x = lbtest.to_dev(xh)
    y = torch.empty((xh.shape[0], b), dtype=torch.float16, device="cuda")
    L.forward(x, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("a,b,s,res", [(4096, 11008, 133, True), (8192, 28672, 256, False),
                                       (1000, 600, 40, True)])
def test_signs_held_once_until_a_batched_forward(lbm, a, b, s, res):
    torch = lbtest.torch_dev()
    say(f"[case] sign storage a={a} b={b} s={s} res={res}")
    paths = lb_synth.layer_inputs(a, b, s, res, seed=s + 3)
    L = lbm.Layer.from_paths(paths)
    P = len(paths)
    sign_bits = P * s * (a + b)          # the factors' bits, [LB2 column] Ch. 1
    sb0, tb0 = L.device_bytes()
    assert sb0 * 8 >= sign_bits
    # padding: rows to 32 (input) and 16 (output), latent columns to 8 and 32
    assert sb0 * 8 <= sign_bits * 1.05 + 8 * 64 * 1024, (sb0, sign_bits)
    for M in (1, 8):
        xh = lb_synth.activations(M, a, seed=M)
        assert_parity(_fwd(torch, L, xh, b).cpu().numpy(), oracle.forward(xh, paths), f"M={M}")
        assert L.device_bytes()[0] == sb0, "an M < 64 forward added sign storage"
    xh = lb_synth.activations(64, a, seed=64)
    assert_parity(_fwd(torch, L, xh, b).cpu().numpy(), oracle.forward(xh, paths), "M=64")
    sb1, tb1 = L.device_bytes()
    assert 0 < sb1 - sb0 <= sb0, "the matrix-core copy holds each sign word once more"
    assert sb1 * 8 <= 2 * sign_bits * 1.05 + 16 * 64 * 1024
    assert tb1 - tb0 == sb1 - sb0
    L.close()


def test_capture_before_prepare_is_refused(lbm):
    """An M >= 64 forward captured before the matrix-core copy exists
    returns LB_ENOTREADY (nothing allocated under capture); after lb_prepare
    the same forward captures and every replay equals the eager result."""
    torch = lbtest.torch_dev()
    say("[case] capture of an unprepared M = 96 forward")
    a, b, s, M = 1000, 600, 40, 96
    paths = lb_synth.layer_inputs(a, b, s, True, seed=17)
    L = lbm.Layer.from_paths(paths)
    sb0 = L.device_bytes()[0]
    xh = lb_synth.activations(M, a, seed=5)
    x = lbtest.to_dev(xh)
    y = torch.zeros((M, b), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        with pytest.raises(lbm.LBError) as ei:
            L.forward(x, y)
        y.add_(0)  # keep the graph non-empty
    assert ei.value.status == lbm.LB_ENOTREADY
    assert "lb_prepare" in lbm.lb_last_error()
    assert L.device_bytes()[0] == sb0
    del g
    L.prepare(M)
    assert L.device_bytes()[0] > sb0
    y2 = torch.zeros((M, b), dtype=torch.float16, device="cuda")
    g2 = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g2):
        L.forward(x, y2)
    torch.cuda.synchronize()
    ref = _fwd(torch, L, xh, b)
    assert_parity(ref.cpu().numpy(), oracle.forward(xh, paths), "eager after prepare")
    for k in range(3):
        y2.zero_()
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y2, ref), f"replay {k}"
    L.close()


def test_repack_after_prepare_updates_the_matrix_core_copy(lbm):
    """lb_pack_signs on a layer whose matrix-core copy exists rebuilds it:
    the M >= 64 forward then follows the new signs, as the M < 64 ones do."""
    torch = lbtest.torch_dev()
    say("[case] re-pack after prepare")
    a, b, s = 700, 500, 37
    paths = lb_synth.layer_inputs(a, b, s, True, seed=21)
    L = lbm.Layer.from_paths(paths)
    L.prepare(64)
    new = lb_synth.layer_inputs(a, b, s, True, seed=22)
    lbm.lb_pack_signs(L.handle, 1, new[1]["su"], new[1]["sv"])
    mixed = [paths[0], dict(paths[1], su=new[1]["su"], sv=new[1]["sv"])]
    for M in (1, 5, 64, 130):
        xh = lb_synth.activations(M, a, seed=M + 40)
        assert_parity(_fwd(torch, L, xh, b).cpu().numpy(), oracle.forward(xh, mixed), f"M={M}")
    L.close()
