"""Pins of the oracle's Joint-ITQ rotation (LittleBit-2 column,
physicalainews.jp, Ch. 2: an orthogonal R between the factors leaves their
product unchanged; R is found by an iterative rotation of the stacked
factors [U; V], 50 steps by default, and absorbed into U and V).

Each test checks the oracle against something other than its own code:
the invariance the page states, orthogonality, the monotone loss that the
alternating minimisation guarantees, closed forms of the Procrustes step
(from matrices built with QR, not with the SVD the oracle calls), exact
recovery of a rotated binary matrix, equivariance under a rotation of the
stacked factors, and exact power-of-two scaling.
"""
import numpy as np
import pytest

import lb_synth
import oracle


def _qr_q(A):
    """Q of a QR factorisation with diag(R) > 0 (so Q is near I when A is)."""
    Q, Rr = np.linalg.qr(A)
    return Q * np.sign(np.diag(Rr))[None, :]


def _orth(rng, s):
    return _qr_q(rng.standard_normal((s, s)))


def _stack(U, V):
    return np.vstack([np.asarray(U, np.float64), np.asarray(V, np.float64)])


@pytest.mark.parametrize("a,b,s", [(120, 90, 16), (40, 300, 33), (64, 64, 1)])
def test_rotation_leaves_the_product_unchanged(a, b, s):
    """(U R)(V R)^T = U V^T and R^T R = I, the fact the page states."""
    U, V = lb_synth.factors(a, b, s, seed=s)
    Ur, Vr, R = oracle.joint_itq(U, V, iters=50)
    np.testing.assert_allclose(R.T @ R, np.eye(s), atol=1e-12)
    ref = U.astype(np.float64) @ V.astype(np.float64).T
    np.testing.assert_allclose(Ur @ Vr.T, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_loss_never_increases():
    """Each B update and each Procrustes update can only lower ||B - X R||^2."""
    U, V = lb_synth.factors(150, 110, 20, seed=4)
    X = _stack(U, V)
    losses = [oracle.itq_loss(X, oracle.joint_itq_rotation(U, V, k)) for k in range(25)]
    for k in range(1, len(losses)):
        assert losses[k] <= losses[k - 1] * (1 + 1e-12), (k, losses[k - 1], losses[k])
    assert losses[-1] < 0.97 * losses[0]


def test_procrustes_closed_forms_and_optimality():
    rng = np.random.default_rng(8)
    s = 6
    d = rng.uniform(0.5, 3.0, s)
    np.testing.assert_allclose(oracle.procrustes_rotation(np.diag(d)), np.eye(s), atol=1e-12)
    Q0 = _orth(rng, s)
    np.testing.assert_allclose(oracle.procrustes_rotation(Q0), Q0, atol=1e-12)
    P0 = _orth(rng, s)
    np.testing.assert_allclose(oracle.procrustes_rotation(P0 @ np.diag(d) @ Q0.T), P0 @ Q0.T,
                               atol=1e-12)
    # optimality against random rotations and small perturbations of the answer
    M = rng.standard_normal((s, s))
    R = oracle.procrustes_rotation(M)
    best = np.sum(M * R)
    for _ in range(200):
        assert np.sum(M * _orth(rng, s)) <= best + 1e-12
    for _ in range(50):
        K = rng.standard_normal((s, s)) * 1e-3
        Qp = _qr_q(np.eye(s) + (K - K.T))
        assert np.sum(M * (R @ Qp)) <= best + 1e-12


def test_recovers_a_rotated_binary_matrix():
    """X = B0 Q: one step from a start near Q^T lands on R = Q^T exactly (zero loss)."""
    rng = np.random.default_rng(9)
    n, s = 300, 8
    B0 = np.where(rng.random((n, s)) < 0.5, -1.0, 1.0)
    Q = _orth(rng, s)
    X = B0 @ Q
    K = rng.standard_normal((s, s)) * 0.02
    E = _qr_q(np.eye(s) + (K - K.T))
    R0 = Q.T @ E
    R = oracle.joint_itq_rotation(X[:180], X[180:], iters=1, R0=R0)
    np.testing.assert_allclose(R, Q.T, atol=1e-12)
    assert oracle.itq_loss(X, R) < 1e-20
    R5 = oracle.joint_itq_rotation(X[:180], X[180:], iters=5, R0=R0)
    np.testing.assert_allclose(R5, Q.T, atol=1e-12)


def test_single_column():
    """s = 1: R = +-1 keeps the start's sign (X^T sign(X R) has the sign of R)."""
    U, V = lb_synth.factors(30, 20, 1, seed=2)
    assert oracle.joint_itq_rotation(U, V, 7)[0, 0] == 1.0
    assert oracle.joint_itq_rotation(U, V, 7, R0=-np.eye(1))[0, 0] == -1.0


def test_equivariant_under_a_rotation_of_the_factors():
    """With X' = X P and R0' = P^T R0 every step gives R' = P^T R."""
    rng = np.random.default_rng(10)
    U, V = lb_synth.factors(90, 70, 12, seed=6)
    P = _orth(rng, 12)
    R0 = _orth(rng, 12)
    R = oracle.joint_itq_rotation(U, V, 6, R0)
    Rp = oracle.joint_itq_rotation(U.astype(np.float64) @ P, V.astype(np.float64) @ P, 6, P.T @ R0)
    np.testing.assert_allclose(Rp, P.T @ R, atol=1e-10)


def test_the_x_stack_order_and_orientation():
    """Swapping U and V stacks the same rows in another order: same R; the
    rows of X multiply R from the left (X R, not R X or X R^T)."""
    U, V = lb_synth.factors(50, 40, 9, seed=12)
    R1 = oracle.joint_itq_rotation(U, V, 8)
    R2 = oracle.joint_itq_rotation(V, U, 8)
    np.testing.assert_allclose(R1, R2, atol=1e-12)
    # one step by hand on a 3 x 2 example: X R0 = X, B = sign(X), X^T B
    X = np.array([[2.0, -1.0], [0.5, 3.0], [-1.0, -0.25]])
    # X^T sign(X) by hand: [[2 + 0.5 + 1, -2 + 0.5 + 1], [-1 + 3 + 0.25, 1 + 3 + 0.25]]
    M = np.array([[3.5, -0.5], [2.25, 4.25]])
    R = oracle.joint_itq_rotation(X[:1], X[1:], 1)
    # polar factor of a 2 x 2 matrix [[p, q], [r, t]] with det > 0: the
    # rotation by atan2(r - q, p + t), which maximises c (p + t) + s (r - q)
    assert np.linalg.det(M) > 0
    th = np.arctan2(M[1, 0] - M[0, 1], M[0, 0] + M[1, 1])
    np.testing.assert_allclose(R, [[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]], atol=1e-12)
    # zeros quantise to +1 (0 and -0 alike): X = [[2, -1], [0, 3], [-1, -0]]
    # gives B = [[1, -1], [1, 1], [-1, 1]] and X^T B = [[3, -3], [2, 4]] by hand
    X0 = np.array([[2.0, -1.0], [0.0, 3.0], [-1.0, -0.0]])
    R = oracle.joint_itq_rotation(X0[:2], X0[2:], 1)
    th = np.arctan2(2.0 - (-3.0), 3.0 + 4.0)
    np.testing.assert_allclose(R, [[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]], atol=1e-12)


@pytest.mark.parametrize("residual", [False, True])
def test_dual_svid_with_itq_scales_exactly(residual):
    """Scaling W by 16 scales the factors by 4, which leaves every sign and R
    unchanged, and scales h and g by 2 and l by 4, exactly."""
    W = lb_synth.weight_matrix(48, 40, seed=13)
    p1 = oracle.dual_svid(W, 6, residual, itq_iters=5)
    p16 = oracle.dual_svid(16.0 * W, 6, residual, itq_iters=5)
    for a, b in zip(p1, p16):
        assert np.array_equal(a["su"], b["su"]) and np.array_equal(a["sv"], b["sv"])
        np.testing.assert_array_equal(b["h"].astype(np.float64), 2.0 * a["h"].astype(np.float64))
        np.testing.assert_array_equal(b["g"].astype(np.float64), 2.0 * a["g"].astype(np.float64))
        np.testing.assert_array_equal(b["l"].astype(np.float64), 4.0 * a["l"].astype(np.float64))


def test_dual_svid_applies_the_rotation_before_binarising():
    """The composition: Dual-SVID with ITQ binarises U R and V R (the rotated
    truncated-SVD factors), and the rotation changes the signs of a generic W."""
    W = lb_synth.weight_matrix(60, 44, seed=14)
    s = 7
    with_itq = oracle.dual_svid(W, s, False, itq_iters=4)[0]
    without = oracle.dual_svid(W, s, False)[0]
    U, V = oracle.svd_factors(W, s)
    R = oracle.joint_itq_rotation(U, V, 4)
    assert np.array_equal(with_itq["su"], oracle.sign_words(U @ R))
    assert np.array_equal(with_itq["sv"], oracle.sign_words(V @ R))
    assert not np.array_equal(with_itq["su"], without["su"])
