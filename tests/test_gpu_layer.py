"""GPU parity of single layers through the C ABI against the float64 oracle.

Bar: relative L2 <= 1e-3 and max |err| <= 1e-2 * rms(y_ref) for fp16
outputs with fp32 accumulation; bit-exact for sign packing and for the
power-of-two scalings that must commute with every fp32 step.
Layer definition: Samsung LittleBit news page (aifrontier.co.jp), Sec. 2.
"""
import numpy as np
import pytest

import lb_synth
import oracle
from tests import lbtest
from tests.lbtest import assert_parity, gpu_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbm():
    lbtest.torch_dev()
    return lbtest.ensure_built()


def _layer(lbm, paths):
    return lbm.Layer.from_paths(paths)


def _check(lbm, a, b, s, res, M, seed, what):
    say(f"[case] {what} a={a} b={b} s={s} residual={res} M={M} seed={seed}")
    paths = lb_synth.layer_inputs(a, b, s, res, seed=seed)
    x = lb_synth.activations(M, a, seed=seed)
    L = _layer(lbm, paths)
    y = gpu_forward(L, x, b)
    ref = oracle.forward(x, paths)
    return assert_parity(y, ref, what), (paths, x, y, L)


def test_tiny_single_path_with_dense_check(lbm):
    """256 -> 256, s = 32, single path, M = 1; also against the dense W."""
    (_, _, _), (paths, x, y, _) = _check(lbm, 256, 256, 32, False, 1, 0, "tiny")
    W = oracle.dense_weight(paths)
    assert_parity(y, x.astype(np.float64) @ W.T, "tiny dense")


def test_llama7b_attention_projection_decode(lbm):
    """4096 -> 4096 at 0.1 BPW (s = 86 per path, residual), M = 1."""
    _check(lbm, 4096, 4096, 86, True, 1, 1, "attn-proj")


@pytest.mark.parametrize("a,b,s,res,M", [
    (100, 37, 5, True, 1), (33, 65, 1, False, 3), (1, 1, 1, True, 1), (257, 129, 63, True, 2),
    (64, 64, 64, False, 1), (96, 200, 65, True, 5), (1000, 3, 33, True, 1), (3, 1000, 31, False, 7),
    (4096, 11008, 133, True, 1), (11008, 4096, 133, True, 1)])
def test_odd_and_mlp_shapes(lbm, a, b, s, res, M):
    _check(lbm, a, b, s, res, M, a + b + s, "odd")


def test_every_M_across_the_path_switch(lbm):
    """M = 1 .. 70 crosses the wave-path / MFMA-path switch at M = 64."""
    a, b, s = 320, 192, 45
    paths = lb_synth.layer_inputs(a, b, s, True, seed=7)
    L = _layer(lbm, paths)
    x_all = lb_synth.activations(70, a, seed=7)
    for M in range(1, 71):
        say(f"[case] M sweep M={M}")
        x = x_all[:M]
        y = gpu_forward(L, x, b)
        assert_parity(y, oracle.forward(x, paths), f"M={M}")


@pytest.mark.parametrize("a,b,s,M", [(4096, 4096, 290, 128), (4096, 11008, 431, 128),
                                     (11008, 4096, 431, 128), (4096, 4096, 290, 200),
                                     (520, 300, 97, 64), (136, 72, 19, 300)])
def test_mfma_path_shapes(lbm, a, b, s, M):
    _check(lbm, a, b, s, True, M, a * 7 + s, "mfma")


@pytest.mark.parametrize("a,b,s,res,M", [(257, 129, 63, False, 65), (1000, 3, 33, True, 64),
                                         (3, 1000, 31, False, 100), (4096, 4096, 86, False, 128),
                                         (33, 65, 1, True, 513)])
def test_mfma_path_odd_shapes(lbm, a, b, s, res, M):
    """Widths and ranks off every tile size, single and residual paths,
    row counts across the 256-row chunking."""
    _check(lbm, a, b, s, res, M, a + 3 * b + s, "mfma-odd")


def test_rows_are_independent(lbm):
    """Row m of a batched call matches the M = 1 call on row m."""
    a, b, s = 512, 256, 40
    paths = lb_synth.layer_inputs(a, b, s, True, seed=9)
    L = _layer(lbm, paths)
    x = lb_synth.activations(128, a, seed=9)
    for M in (7, 128):
        say(f"[case] row independence M={M}")
        yb = gpu_forward(L, x[:M], b)
        for m in (0, M // 2, M - 1):
            y1 = gpu_forward(L, x[m:m + 1], b)
            assert_parity(yb[m:m + 1], y1.astype(np.float64), f"row {m} of M={M}")


def test_pack_unpack_bit_exact_and_padding_ignored(lbm):
    a, b, s = 200, 100, 45
    paths = lb_synth.layer_inputs(a, b, s, True, seed=11)
    junk = [dict(p, su=lb_synth.garbage_padding(p["su"], s, 1), sv=lb_synth.garbage_padding(p["sv"], s, 2))
            for p in paths]
    Lc = _layer(lbm, paths)
    Lj = _layer(lbm, junk)
    for p in range(2):
        su, sv = lbm.lb_unpack_signs(Lc.handle, p)
        assert np.array_equal(su, paths[p]["su"]) and np.array_equal(sv, paths[p]["sv"])
        su, sv = lbm.lb_unpack_signs(Lj.handle, p)
        assert np.array_equal(su, paths[p]["su"]) and np.array_equal(sv, paths[p]["sv"])
    x = lb_synth.activations(3, a, seed=11)
    assert np.array_equal(gpu_forward(Lc, x, b).view(np.uint16), gpu_forward(Lj, x, b).view(np.uint16))
    x64 = lb_synth.activations(64, a, seed=12)
    assert np.array_equal(gpu_forward(Lc, x64, b).view(np.uint16), gpu_forward(Lj, x64, b).view(np.uint16))


@pytest.mark.parametrize("M", [1, 5, 64, 96])
def test_zero_input_gives_exact_zero(lbm, M):
    a, b, s = 300, 130, 37
    L = _layer(lbm, lb_synth.layer_inputs(a, b, s, True, seed=13))
    y = gpu_forward(L, np.zeros((M, a), np.float16), b)
    assert (y.astype(np.float64) == 0).all()


@pytest.mark.parametrize("which", ["h", "g", "l"])
@pytest.mark.parametrize("M", [1, 3, 80])
def test_power_of_two_scaling_is_bit_exact(lbm, which, M):
    a, b, s = 384, 160, 50
    paths = lb_synth.layer_inputs(a, b, s, True, seed=14)
    x = lb_synth.activations(M, a, seed=14)
    twice = [dict(p, **{which: (p[which].astype(np.float64) * 2).astype(np.float16)}) for p in paths]
    y1 = gpu_forward(_layer(lbm, paths), x, b).astype(np.float32)
    y2 = gpu_forward(_layer(lbm, twice), x, b).astype(np.float32)
    assert np.array_equal(2 * y1, y2)


@pytest.mark.parametrize("M", [1, 70])
def test_residual_is_sum_of_single_paths(lbm, M):
    a, b, s = 640, 320, 33
    paths = lb_synth.layer_inputs(a, b, s, True, seed=15)
    x = lb_synth.activations(M, a, seed=15)
    y = gpu_forward(_layer(lbm, paths), x, b).astype(np.float64)
    y0 = gpu_forward(_layer(lbm, paths[:1]), x, b).astype(np.float64)
    y1 = gpu_forward(_layer(lbm, paths[1:]), x, b).astype(np.float64)
    assert_parity(y, y0 + y1, "residual sum")


@pytest.mark.parametrize("M", [1, 128])
def test_run_to_run_bitwise_determinism(lbm, M):
    a, b, s = 4096, 4096, 86
    paths = lb_synth.layer_inputs(a, b, s, True, seed=16)
    L = _layer(lbm, paths)
    x = lb_synth.activations(M, a, seed=16)
    ys = [gpu_forward(L, x, b).view(np.uint16) for _ in range(3)]
    assert all(np.array_equal(ys[0], v) for v in ys[1:])


def test_split_stages_match_the_definition(lbm):
    torch = lbtest.torch_dev()
    a, b, s = 700, 260, 29
    paths = lb_synth.layer_inputs(a, b, s, True, seed=17)
    L = _layer(lbm, paths)
    for M in (1, 9, 70):
        say(f"[case] split stages M={M}")
        x = lb_synth.activations(M, a, seed=M)
        xd = lbtest.to_dev(x)
        w = torch.empty((M, 2 * s), dtype=torch.float32, device="cuda")
        y = torch.empty((M, b), dtype=torch.float16, device="cuda")
        lbm.lb_forward_stage1(L.handle, xd, w, M)
        lbm.lb_forward_stage2(L.handle, w, y, M)
        torch.cuda.synchronize()
        wg = w.cpu().numpy()
        assert_parity(wg, oracle.latent(x, paths), "latent w")
        assert_parity(y.cpu().numpy(), oracle.forward(x, paths), "stage2 output")
        # the second half alone: the oracle's product from the GPU's own latent
        assert_parity(y.cpu().numpy(), oracle.from_latent(wg, paths), "stage2 from the GPU latent")


def test_error_codes(lbm):
    torch = lbtest.torch_dev()
    L = lbm.Layer(64, 32, 8, True)
    p0 = lb_synth.path_inputs(64, 32, 8, seed=1)
    x = torch.zeros((2, 64), dtype=torch.float16, device="cuda")
    y = torch.zeros((2, 32), dtype=torch.float16, device="cuda")
    with pytest.raises(lbm.LBError) as ei:
        L.forward(x, y)
    assert ei.value.status == lbm.LB_ENOTREADY
    lbm.lb_pack_signs(L.handle, 0, p0["su"], p0["sv"])
    lbm.lb_set_scales(L.handle, 0, p0["h"], p0["g"], p0["l"])
    with pytest.raises(lbm.LBError) as ei:   # path 1 still missing
        L.forward(x, y)
    assert ei.value.status == lbm.LB_ENOTREADY
    lbm.lb_pack_signs(L.handle, 1, p0["su"], p0["sv"])
    lbm.lb_set_scales(L.handle, 1, p0["h"], p0["g"], p0["l"])
    L.forward(x, y)
    lbm.lb_forward(L.handle, x, y, 0)        # M = 0 is a no-op
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_pack_signs(L.handle, 2, p0["su"], p0["sv"])
    assert ei.value.status == lbm.LB_EINVAL
    big = torch.zeros((4, 64), dtype=torch.float16, device="cuda").view(-1)
    with pytest.raises(lbm.LBError) as ei:   # y (64 bytes in) overlaps x's first row
        lbm.lb_forward(L.handle, big, big[32:], 1)
    assert ei.value.status == lbm.LB_EINVAL
    with pytest.raises(lbm.LBError) as ei:   # misaligned x
        lbm.lb_forward(L.handle, x.data_ptr() + 2, y, 1)
    assert ei.value.status == lbm.LB_EINVAL
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_forward(L.handle, x, y, -1)
    assert ei.value.status == lbm.LB_EINVAL
    torch.cuda.synchronize()


def test_eff_bits_and_rank_from_the_gpu_build(lbm):
    from fractions import Fraction
    n, d = lbm.lb_eff_bits(256, 256, 32, False)
    assert Fraction(n, d) == Fraction(49, 128)
    assert lbm.lb_rank_for_bpw(8192, 28672, 1, 10, True) == 302
