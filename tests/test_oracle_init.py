"""Pins of the oracle's initialisation from real factors ([LB news] Sec. 2,
Dual-SVID: factor signs from a truncated SVD, magnitudes turned into the
h, g, l scales by a rank-1 approximation).

Each test checks the oracle against something other than its own code: a
plain-Python bit reader, closed forms for exactly rank-1 magnitudes, the
Eckart-Young error identities, an independent power iteration, and exact
power-of-two scaling.
"""
import math

import numpy as np
import pytest

import oracle


def _bit(words, r, k):
    return (int(words[r][k // 32]) >> (k % 32)) & 1


def test_sign_words_bit_by_bit_zero_is_plus():
    rng = np.random.default_rng(1)
    F = rng.standard_normal((7, 45))
    F[0, 3] = 0.0
    F[2, 40] = -0.0
    F[5, 31] = -1e-300
    words = oracle.sign_words(F)
    assert words.shape == (7, 2) and words.dtype == np.uint32
    for r in range(7):
        for k in range(45):
            x = float(F[r, k])
            want = 0 if (x < 0.0) else 1      # -0.0 < 0.0 is False: sign(-0) = +1
            assert _bit(words, r, k) == want, (r, k, x)
        for k in range(45, 64):               # padding bits are zero
            assert _bit(words, r, k) == 0


def test_rank1_of_an_exact_rank1_magnitude():
    rng = np.random.default_rng(2)
    r0 = rng.uniform(0.2, 3.0, 33)
    c0 = rng.uniform(0.1, 2.0, 17)
    signs = np.where(rng.random((33, 17)) < 0.5, -1.0, 1.0)
    r, c = oracle.rank1_magnitude(signs * np.outer(r0, c0))
    assert (r >= 0).all() and (c >= 0).all()
    np.testing.assert_allclose(np.outer(r, c), np.outer(r0, c0), rtol=1e-12, atol=0)
    # the even split: |r| = |c| * (|r0| |c0| / |c|^2), i.e. ||r|| = ||c||
    assert math.isclose(np.linalg.norm(r), np.linalg.norm(c), rel_tol=1e-12)


def _power_iteration(A, iters=500):
    """Independent top singular pair of a nonnegative matrix, plain loops."""
    v = np.ones(A.shape[1]) / math.sqrt(A.shape[1])
    for _ in range(iters):
        u = A @ v
        v = A.T @ u
        v = v / np.linalg.norm(v)
    u = A @ v
    sig = np.linalg.norm(u)
    return u / math.sqrt(sig), v * math.sqrt(sig)


def test_rank1_matches_power_iteration_and_eckart_young():
    rng = np.random.default_rng(3)
    F = rng.standard_normal((60, 24)) * rng.uniform(0.5, 2.0, 24)[None, :]
    A = np.abs(F)
    r, c = oracle.rank1_magnitude(F)
    pr, pc = _power_iteration(A)
    np.testing.assert_allclose(np.outer(r, c), np.outer(pr, pc), rtol=1e-9, atol=1e-12)
    # best rank-1: the squared error is ||A||^2 - sigma_1^2 with sigma_1 = ||r|| ||c||
    err2 = np.linalg.norm(A - np.outer(r, c)) ** 2
    sig1 = np.linalg.norm(r) * np.linalg.norm(c)
    assert math.isclose(err2, np.linalg.norm(A) ** 2 - sig1 ** 2, rel_tol=1e-9)
    # and no other rank-1 candidate does better
    for rr, cc in [(A.mean(1), np.ones(24)), (r * 1.01, c), (r, c + 0.01), (A[:, 0], A[0] / A[0, 0])]:
        assert np.linalg.norm(A - np.outer(rr, cc)) >= math.sqrt(err2) - 1e-12


def test_init_reconstructs_factors_with_rank1_magnitudes():
    """|U| = outer(h0, lu0) and |V| = outer(g0, lv0) exactly: the unrounded
    scales reproduce U V^T = diag(h) S_U diag(l) S_V^T diag(g)."""
    rng = np.random.default_rng(4)
    b, a, s = 23, 19, 11
    h0, lu0 = rng.uniform(0.5, 1.5, b), rng.uniform(0.5, 1.5, s)
    g0, lv0 = rng.uniform(0.5, 1.5, a), rng.uniform(0.5, 1.5, s)
    U = np.where(rng.random((b, s)) < 0.5, -1.0, 1.0) * np.outer(h0, lu0)
    V = np.where(rng.random((a, s)) < 0.5, -1.0, 1.0) * np.outer(g0, lv0)
    p = oracle.init_from_factors(U, V, round_fp16=False)
    S_U = oracle.unpack_signs(p["su"], s).astype(np.float64)
    S_V = oracle.unpack_signs(p["sv"], s).astype(np.float64)
    W_hat = (p["h"][:, None] * S_U * p["l"][None, :]) @ (S_V * p["g"][:, None]).T
    np.testing.assert_allclose(W_hat, U @ V.T, rtol=1e-11, atol=1e-12)
    # rounded scales are the fp16 (RNE) of the unrounded ones
    q = oracle.init_from_factors(U, V)
    for k in ("h", "g", "l"):
        assert q[k].dtype == np.float16
        np.testing.assert_array_equal(q[k], p[k].astype(np.float16))


def test_svd_factors_truncation_identities():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((30, 20))
    sv = np.linalg.svd(W, compute_uv=False)
    for s in (1, 5, 20):
        Up, Vp = oracle.svd_factors(W, s)
        assert Up.shape == (30, s) and Vp.shape == (20, s)
        err2 = np.linalg.norm(W - Up @ Vp.T) ** 2
        assert math.isclose(err2, float((sv[s:] ** 2).sum()), rel_tol=1e-9, abs_tol=1e-20)
        # the singular values are split evenly: U'^T U' = V'^T V' = diag(sigma)
        np.testing.assert_allclose(Up.T @ Up, np.diag(sv[:s]), atol=1e-10)
        np.testing.assert_allclose(Vp.T @ Vp, np.diag(sv[:s]), atol=1e-10)
    # a rank-4 W is reproduced exactly from 4 factors
    W4 = rng.standard_normal((30, 4)) @ rng.standard_normal((4, 20))
    Up, Vp = oracle.svd_factors(W4, 4)
    np.testing.assert_allclose(Up @ Vp.T, W4, atol=1e-12)


@pytest.mark.parametrize("residual", [False, True])
def test_dual_svid_commutes_with_power_of_two_scaling(residual):
    rng = np.random.default_rng(6)
    W = rng.standard_normal((24, 36))
    # W -> 16 W: singular values x16, factors x4, |factors| x4, the even
    # rank-1 split gives h, g x2 and l = l_u l_v x4: all powers of two, so
    # the fp16 scales, the residual and every sign scale exactly
    p1 = oracle.dual_svid(W, 6, residual)
    p16 = oracle.dual_svid(16.0 * W, 6, residual)
    assert len(p1) == (2 if residual else 1)
    for q1, q16 in zip(p1, p16):
        np.testing.assert_array_equal(q1["su"], q16["su"])
        np.testing.assert_array_equal(q1["sv"], q16["sv"])
        np.testing.assert_array_equal(q16["h"], 2 * q1["h"])
        np.testing.assert_array_equal(q16["g"], 2 * q1["g"])
        np.testing.assert_array_equal(q16["l"], 4 * q1["l"])
    np.testing.assert_array_equal(oracle.dense_weight(p16), 16.0 * oracle.dense_weight(p1))


def test_dual_svid_residual_path_fits_what_the_main_path_left():
    """The residual path's factors are those of W minus the main path's
    dense weight: on a W that the main path reproduces exactly (rank-1
    magnitudes, fp16-exact scales), the residual starts from zero."""
    b, a, s = 8, 6, 2
    U = np.array([[1, -1], [2, 2], [-1, 1], [2, -2], [1, 1], [-2, 2], [1, -1], [2, 2]], float) * np.array([1.0, 0.5])
    V = np.array([[1, 1], [-2, 2], [1, -1], [2, 2], [-1, -1], [2, -2]], float) * np.array([1.0, 0.5])
    W = U @ V.T
    main = oracle.init_from_factors(*oracle.svd_factors(W, s))
    left = W - oracle.dense_weight([main])
    paths = oracle.dual_svid(W, s, True)
    np.testing.assert_array_equal(paths[0]["su"], main["su"])
    assert np.linalg.norm(oracle.dense_weight(paths) - W) <= np.linalg.norm(left) + 1e-12
