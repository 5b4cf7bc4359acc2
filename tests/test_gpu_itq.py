"""GPU parity of the Joint-ITQ rotation through the C ABI (LittleBit-2
column, physicalainews.jp, Ch. 2: an orthogonal R between the factors
leaves their product unchanged; R comes from an iterative rotation of the
stacked factors [U; V], 50 steps by default, and is absorbed into U and V
before binarising).

Bar: the device rotation within 1e-9 (max abs) of the oracle's after the
same number of steps from the same start (both fp64; the device's polar
factor is a Newton-Schulz iteration run to 1e-12, the oracle's an SVD), the
codes sign(X R) identical; a path set from rotated factors: sign words
bit-exact and scales within one fp16 step of the oracle given the same R;
the whole Dual-SVID + Joint-ITQ recipe at the forward bar.
"""
import numpy as np
import pytest

import lb_synth
import oracle
from tests import lbtest
from tests.lbtest import assert_parity, gpu_forward, say
from tests.test_gpu_init import _compare_path, _key

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbm():
    lbtest.torch_dev()
    return lbtest.ensure_built()


def _dev(x):
    return lbtest.to_dev(np.ascontiguousarray(x))


def _orth(rng, s):
    Q, Rr = np.linalg.qr(rng.standard_normal((s, s)))
    return Q * np.sign(np.diag(Rr))[None, :]


def _itq(lbm, U, V, iters, R0=None):
    R = lbm.lb_joint_itq(_dev(U), _dev(V), iters, None if R0 is None else _dev(R0))
    return R.cpu().numpy()


@pytest.mark.parametrize("a,b,s,iters", [
    (120, 90, 16, 50), (40, 300, 33, 50), (64, 64, 1, 7), (257, 129, 63, 50), (1, 1, 1, 3),
    (1000, 3, 5, 20), (4096, 4096, 86, 50), (8192, 28672, 302, 50)])
def test_itq_matches_oracle(lbm, a, b, s, iters):
    say(f"[case] itq a={a} b={b} s={s} iters={iters}")
    U, V = lb_synth.factors(a, b, s, seed=a + 2 * b + s)
    R = _itq(lbm, U, V, iters)
    ref = oracle.joint_itq_rotation(U, V, iters)
    err = float(np.abs(R - ref).max())
    X = np.vstack([U, V]).astype(np.float64)
    flips = int(np.count_nonzero(oracle.sign_pm1(X @ R) != oracle.sign_pm1(X @ ref)))
    say(f"  max |R - R_ref| = {err:.3e}, code flips {flips}")
    assert err <= 1e-9
    assert flips == 0
    np.testing.assert_allclose(R.T @ R, np.eye(s), atol=1e-11)


def test_itq_from_a_start_rotation(lbm):
    rng = np.random.default_rng(3)
    a, b, s = 200, 150, 24
    say(f"[case] itq start rotation a={a} b={b} s={s}")
    U, V = lb_synth.factors(a, b, s, seed=17)
    R0 = _orth(rng, s)
    for iters in (0, 1, 10):
        R = _itq(lbm, U, V, iters, R0)
        ref = oracle.joint_itq_rotation(U, V, iters, R0)
        assert np.abs(R - ref).max() <= 1e-9, iters
    assert np.array_equal(_itq(lbm, U, V, 0), np.eye(s))


def test_itq_recovers_a_rotated_binary_matrix(lbm):
    """X = B0 Q from a start near Q^T: one step gives R = Q^T (as the oracle pin)."""
    rng = np.random.default_rng(9)
    n, s = 300, 8
    B0 = np.where(rng.random((n, s)) < 0.5, -1.0, 1.0)
    Q = _orth(rng, s)
    X = (B0 @ Q).astype(np.float32)
    K = rng.standard_normal((s, s)) * 0.02
    E, Rr = np.linalg.qr(np.eye(s) + (K - K.T))
    E = E * np.sign(np.diag(Rr))[None, :]
    R = _itq(lbm, X[:180], X[180:], 1, Q.T @ E)
    Xd = X.astype(np.float64)
    assert np.array_equal(oracle.sign_pm1(Xd @ R), B0)
    np.testing.assert_allclose(R, oracle.joint_itq_rotation(X[:180], X[180:], 1, Q.T @ E),
                               atol=1e-12)


def test_itq_is_deterministic(lbm):
    U, V = lb_synth.factors(2048, 1536, 70, seed=5)
    say("[case] itq determinism")
    R1 = _itq(lbm, U, V, 20)
    R2 = _itq(lbm, U, V, 20)
    assert np.array_equal(R1.view(np.uint8), R2.view(np.uint8))


@pytest.mark.parametrize("a,b,s", [(100, 70, 12), (257, 129, 63), (8192, 28672, 302)])
def test_init_from_rotated_factors(lbm, a, b, s):
    """The path from U R and V R, with the oracle's rotation given to both sides."""
    say(f"[case] init rotated a={a} b={b} s={s}")
    U, V = lb_synth.factors(a, b, s, seed=s + 1)
    R = oracle.joint_itq_rotation(U, V, 5)
    Ur, Vr = U.astype(np.float64) @ R, V.astype(np.float64) @ R
    ref = oracle.init_from_factors(Ur, Vr)
    L = lbm.Layer(a, b, s, False)
    lbm.lb_init_from_factors(L.handle, 0, _dev(U), _dev(V), _dev(R))
    _compare_path(lbm, L, 0, ref, f"rotated {a}x{b}x{s}")
    x = lb_synth.activations(2, a, seed=8)
    assert_parity(gpu_forward(L, x, b), oracle.forward(x, [dict(ref, a=a, b=b)]), "rotated fwd")


def test_dual_svid_with_joint_itq(lbm):
    """SVD (numpy, a library routine, on the caller's side), Joint-ITQ and the
    init on the device, for both paths; against oracle.dual_svid with ITQ."""
    a, b, s, iters = 512, 384, 40, 50
    say(f"[case] dual-svid + joint-itq a={a} b={b} s={s}")
    W = lb_synth.weight_matrix(a, b, seed=31)

    def svd_factors(Wm):
        Uf, S, Vt = np.linalg.svd(Wm, full_matrices=False)
        r = np.sqrt(S[:s])
        return (Uf[:, :s] * r).astype(np.float32), (Vt[:s].T * r).astype(np.float32)

    L = lbm.Layer(a, b, s, True)
    for p in range(2):
        if p == 0:
            Wm = W
        else:
            su, sv = lbm.lb_unpack_signs(L.handle, 0)
            h, g, l = lbm.lb_get_scales(L.handle, 0)
            Wm = W - oracle.dense_weight([{"s": s, "su": su, "sv": sv, "h": h, "g": g, "l": l}])
        Uf, Vf = svd_factors(Wm)
        Ud, Vd = _dev(Uf), _dev(Vf)
        R = lbm.lb_joint_itq(Ud, Vd, iters)
        lbm.lb_init_from_factors(L.handle, p, Ud, Vd, R)

    ref = oracle.dual_svid(W, s, residual=True, itq_iters=iters)
    for p in range(2):
        su, sv = lbm.lb_unpack_signs(L.handle, p)
        agree = [np.mean(oracle.unpack_signs(x, s) == oracle.unpack_signs(ref[p][k], s))
                 for x, k in ((su, "su"), (sv, "sv"))]
        say(f"  path {p}: sign agreement {agree[0]:.6f} {agree[1]:.6f}")
        assert min(agree) >= 0.999
        h, g, l = lbm.lb_get_scales(L.handle, p)
        for v, k in ((h, "h"), (g, "g"), (l, "l")):
            assert np.mean(np.abs(_key(v) - _key(ref[p][k])) <= 1) >= 0.999, f"path {p} {k}"
    x = lb_synth.activations(4, a, seed=32)
    paths = [dict(r, a=a, b=b) for r in ref]
    assert_parity(gpu_forward(L, x, b), oracle.forward(x, paths), "dual-svid + itq forward")


def test_itq_argument_errors(lbm):
    torch = lbtest.torch_dev()
    U = torch.zeros((8, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        lbm.lb_joint_itq(U, U, 5, R0=torch.eye(3, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        lbm.lb_joint_itq(U.double(), U, 5)


def test_itq_zero_factors_are_rejected(lbm):
    """X = 0 makes X^T B = 0, whose polar factor is not defined: LB_EUNSUPPORTED."""
    torch = lbtest.torch_dev()
    say("[case] itq zero factors")
    Z = torch.zeros((6, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(lbm.LBError) as ei:
        lbm.lb_joint_itq(Z, Z, 2)
    assert ei.value.status == lbm.LB_EUNSUPPORTED
