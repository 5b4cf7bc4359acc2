"""Float64 CPU oracle for the LittleBit factorized binary linear forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it, and it shares no code with the HIP library.

Sources (the web pages this method is taken from; cited by short name):

* [LB2 column] physicalainews.jp, "LittleBit-2: sub-1-bit LLM quantization
  (2026)".  Ch. 1 defines the effective bit width of a LittleBit layer
  (one formula without and one with the residual path); Ch. 2 describes
  the binary low-rank factors and the Joint-ITQ rotation.
* [LB news] aifrontier.co.jp, "Samsung LittleBit: 13B to 0.84 GB".  Sec. 1
  has the model-size table; Sec. 2 ("how it works") says the weight matrix
  is approximated by the product of two binarised (+-1) low-rank factors,
  with three learnable FP16 scales (row h, column g, latent l), that the
  residual path is a second factorisation whose output is added at
  inference, and that inference is two small binary matrix products plus
  elementwise scaling.

Readings where the pages are silent (each one is also listed in the
design notes):

* polarity: bit 1 is +1 and bit 0 is -1;
* canonical packing: each row of S_U (b x s) and of S_V (a x s) is packed
  along s, 32 entries per uint32, entry k in bit k % 32 of word k // 32;
  bits past s are ignored;
* orientation: a is the input width and b the output width, W is b x a and
  W ~= diag(h) S_U diag(l) S_V^T diag(g);
* residual: both paths read the same x, have fully independent
  (S_U, S_V, h, g, l) and are summed;
* no bias (the bit count of [LB2 column] Ch. 1 has no bias term).

Every function here is pinned by tests that do not re-type it: brute-force
loops on tiny inputs, closed forms, invariants, hand-worked fixtures under
``tests/golden/`` and the model sizes printed in [LB news] Sec. 1.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "unpack_signs", "pack_signs", "num_bits", "eff_bits", "rank_for_bpw",
    "forward", "forward_path", "latent", "from_latent", "dense_weight", "combine", "stack_units",
    "sign_words", "rank1_magnitude", "init_from_factors", "svd_factors", "dual_svid",
    "sign_pm1", "procrustes_rotation", "itq_loss", "joint_itq_rotation", "joint_itq",
]


# --------------------------------------------------------------------------
# Sign bits
# --------------------------------------------------------------------------
def unpack_signs(words, s: int) -> np.ndarray:
    """Canonical words (rows x ceil(s/32) uint32) -> +-1 int8 matrix (rows x s).

    [LB news] Sec. 2: the factors are binarised to +-1 and stored as bits.
    Bits past ``s`` in the last word are ignored.
    """
    words = np.ascontiguousarray(words, dtype=np.uint32)
    rows = words.shape[0]
    out = np.empty((rows, s), dtype=np.int8)
    for k in range(s):
        bit = (words[:, k // 32] >> np.uint32(k % 32)) & np.uint32(1)
        out[:, k] = np.where(bit == 1, 1, -1)
    return out


def pack_signs(S) -> np.ndarray:
    """+-1 matrix (rows x s) -> canonical words (rows x ceil(s/32) uint32).

    Padding bits are zero.  Inverse of :func:`unpack_signs`.
    """
    S = np.asarray(S)
    rows, s = S.shape
    words = np.zeros((rows, (s + 31) // 32), dtype=np.uint32)
    for k in range(s):
        one = (S[:, k] > 0).astype(np.uint32)
        words[:, k // 32] |= one << np.uint32(k % 32)
    return words


# --------------------------------------------------------------------------
# Bit accounting ([LB2 column] Ch. 1)
# --------------------------------------------------------------------------
def num_bits(a: int, b: int, s: int, residual: bool) -> int:
    """Storage bits of one layer: s*(a+b+16) + 16*(a+b) per path.

    [LB2 column] Ch. 1 gives the single-path count and the residual count,
    which doubles every term.  a = input width, b = output width, s = rank.
    """
    paths = 2 if residual else 1
    return paths * (s * (a + b + 16) + 16 * (a + b))


def eff_bits(a: int, b: int, s: int, residual: bool) -> Fraction:
    """Effective bits per weight, exactly: num_bits / (a*b) ([LB2 column] Ch. 1)."""
    return Fraction(num_bits(a, b, s, residual), a * b)


def rank_for_bpw(a: int, b: int, bpw, residual: bool) -> int:
    """Largest rank s whose effective bit width does not exceed ``bpw``.

    Solves the bit count of [LB2 column] Ch. 1 for s in exact rationals and
    takes the floor.  Raises ValueError when even s = 0 exceeds the budget.
    """
    bpw = Fraction(bpw)
    paths = 2 if residual else 1
    budget = bpw * a * b - 16 * paths * (a + b)
    if budget < 0:
        raise ValueError("bit budget too small for the scale vectors alone")
    return int(budget // (paths * (a + b + 16)))


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def _f64(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float16).astype(np.float64)


def forward_path(x, path: dict) -> np.ndarray:
    """One path: h * (S_U (l * (S_V^T (g * x)))), rows of x independent.

    [LB news] Sec. 2: two small binary matrix products and elementwise
    scaling with the column scale g, latent scale l and row scale h.
    ``x`` is (M x a) fp16; the result is float64 (M x b), not rounded.
    """
    s = path["s"]
    S_U = unpack_signs(path["su"], s).astype(np.float64)   # b x s
    S_V = unpack_signs(path["sv"], s).astype(np.float64)   # a x s
    x = _f64(x)
    z = x * _f64(path["g"])[None, :]          # column scale
    t = z @ S_V                               # first binary product
    w = t * _f64(path["l"])[None, :]          # latent scale
    u = w @ S_U.T                             # second binary product
    return u * _f64(path["h"])[None, :]       # row scale


def forward(x, paths) -> np.ndarray:
    """Layer output in float64: the sum of its paths ([LB news] Sec. 2, residual)."""
    y = None
    for p in paths:
        v = forward_path(x, p)
        y = v if y is None else y + v
    return y


def latent(x, paths) -> np.ndarray:
    """The layer's latent vector: w_p = l_p * (S_V,p^T (g_p * x)) for each path,
    placed path-major (columns p*s .. p*s + s - 1 belong to path p), float64.

    [LB news] Sec. 2: the first binary product and the latent scale, which
    is where a cache of factorised K/V projections would keep its entries
    ([LB news] Sec. 4).  ``x`` is (M x a) fp16; the result is (M x P*s).
    """
    cols = []
    x = _f64(x)
    for p in paths:
        S_V = unpack_signs(p["sv"], p["s"]).astype(np.float64)   # a x s
        t = (x * _f64(p["g"])[None, :]) @ S_V                     # first binary product
        cols.append(t * _f64(p["l"])[None, :])                    # latent scale
    return np.concatenate(cols, axis=1)


def from_latent(w, paths) -> np.ndarray:
    """The second half of the layer: y = sum_p h_p * (S_U,p w_p) for a latent
    ``w`` (M x P*s, path-major, any float type), float64 (M x b).

    [LB news] Sec. 2: the second binary product and the row scale; the
    paths are summed.  from_latent(latent(x)) is the forward of x.
    """
    w = np.asarray(w, dtype=np.float64)
    y = None
    off = 0
    for p in paths:
        s = p["s"]
        S_U = unpack_signs(p["su"], s).astype(np.float64)   # b x s
        v = (w[:, off:off + s] @ S_U.T) * _f64(p["h"])[None, :]
        y = v if y is None else y + v
        off += s
    return y


def dense_weight(paths) -> np.ndarray:
    """Dense W (b x a) = sum_p diag(h) S_U diag(l) S_V^T diag(g), float64."""
    W = None
    for p in paths:
        s = p["s"]
        S_U = unpack_signs(p["su"], s).astype(np.float64)
        S_V = unpack_signs(p["sv"], s).astype(np.float64)
        Wp = (_f64(p["h"])[:, None] * S_U) @ (_f64(p["l"])[:, None] * (S_V * _f64(p["g"])[:, None]).T)
        W = Wp if W is None else W + Wp
    return W


# --------------------------------------------------------------------------
# Initialisation from real factors ([LB news] Sec. 2, Dual-SVID)
#
# The page gives one line: the factor signs come from a truncated SVD and
# the magnitudes are turned into scales by a rank-1 approximation.
# Readings (each also listed in the design notes):
# * the singular values are split evenly between the factors,
#   U' = U sqrt(Sigma), V' = V sqrt(Sigma), so that W ~= U' V'^T;
# * sign(0) = +1 (bit 1), for -0.0 as well;
# * the rank-1 approximation of a magnitude matrix is its top singular pair
#   (Eckart-Young), split evenly: |U'| ~= r c^T with r = u sqrt(sigma),
#   c = v sqrt(sigma), both nonnegative;
# * |U'| gives the row scale h and a latent factor l_u, |V'| gives the
#   column scale g and l_v, and l = l_u * l_v, so that
#   U' V'^T ~= diag(h) S_U diag(l) S_V^T diag(g);
# * the residual path takes the same steps on W minus the main path's
#   dense weight (with its fp16 scales).
# --------------------------------------------------------------------------
def sign_words(F) -> np.ndarray:
    """Canonical words of the signs of a real factor (rows x s); 0 and -0 count as +1."""
    F = np.asarray(F, dtype=np.float64)
    return pack_signs(np.where(F >= 0.0, 1, -1))


def rank1_magnitude(F):
    """Top singular pair of |F| (rows x s) as r (rows) and c (s), |F| ~= outer(r, c).

    The pair is the best rank-1 approximation in the Frobenius norm
    (np.linalg.svd is the textbook routine); a nonnegative matrix has a
    nonnegative top pair, whose sign the SVD leaves open and which is fixed
    here so that r and c are >= 0.  The singular value is split evenly.
    """
    A = np.abs(np.asarray(F, dtype=np.float64))
    U, S, Vt = np.linalg.svd(A, full_matrices=False)
    u, v, sig = U[:, 0], Vt[0], float(S[0])
    if u.sum() < 0:
        u, v = -u, -v
    return u * np.sqrt(sig), v * np.sqrt(sig)


def init_from_factors(U, V, round_fp16: bool = True) -> dict:
    """One path from real factors U (b x s) and V (a x s), W ~= U V^T.

    Signs of the factors, h and l_u from the rank-1 fit of |U|, g and l_v
    from that of |V|, l = l_u * l_v.  The scales are rounded to fp16 (RNE)
    unless ``round_fp16`` is False (then they stay float64).
    """
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    h, lu = rank1_magnitude(U)
    g, lv = rank1_magnitude(V)
    l = lu * lv
    cast = (lambda v: v.astype(np.float16)) if round_fp16 else (lambda v: v)
    return {"s": U.shape[1], "su": sign_words(U), "sv": sign_words(V),
            "h": cast(h), "g": cast(g), "l": cast(l)}


def svd_factors(W, s: int):
    """Rank-s truncated SVD of W (b x a) as U' = U sqrt(Sigma) (b x s) and V' (a x s)."""
    W = np.asarray(W, dtype=np.float64)
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    r = np.sqrt(S[:s])
    return U[:, :s] * r[None, :], Vt[:s].T * r[None, :]


def dual_svid(W, s: int, residual: bool, itq_iters: int = 0) -> list:
    """Dual-SVID initialisation of a layer from a real W (b x a), rank s per path.

    With ``itq_iters`` > 0 each path's factors are first rotated by the
    Joint-ITQ rotation of that many steps (started from the identity), as
    LittleBit-2 does before binarising ([LB2 column] Ch. 2).
    """
    W = np.asarray(W, dtype=np.float64)

    def one_path(Wm):
        U, V = svd_factors(Wm, s)
        if itq_iters > 0:
            U, V, _ = joint_itq(U, V, itq_iters)
        return init_from_factors(U, V)

    paths = [one_path(W)]
    if residual:
        paths.append(one_path(W - dense_weight(paths)))
    return paths


# --------------------------------------------------------------------------
# Joint-ITQ rotation ([LB2 column] Ch. 2)
#
# The page states: an orthogonal R (R^T R = I) inserted between the factors
# leaves their product unchanged, (U R)(R^T V^T) = U V^T; LittleBit-2 stacks
# the factors as X = [U; V] (its code concatenates U and the transpose of
# its s x a V along rows, which is our a x s V), finds R by an iterative
# rotation (50 steps by default), rotates both factors with it before
# binarising, and the rotation costs nothing at inference.
# Readings (each also listed in the design notes):
# * "iterative rotation" is iterative quantization (ITQ): minimise the
#   quantisation loss ||B - X R||_F^2 over B in {+-1}^((b+a) x s) and
#   orthogonal R by alternating B = sign(X R) and the R that is optimal for
#   that B, the orthogonal Procrustes solution R = P Q^T for
#   X^T B = P S Q^T;
# * one step = one B update followed by one R update, starting from
#   R0 = I (the page names no start; a caller may pass its own);
# * sign(0) = +1, as for the factor signs;
# * U <- U R and V <- V R in our a x s layout (the page's V <- R^T V).
# --------------------------------------------------------------------------
def sign_pm1(A) -> np.ndarray:
    """+1 where A >= 0 (0 and -0 included), -1 elsewhere, float64."""
    return np.where(np.asarray(A, dtype=np.float64) >= 0.0, 1.0, -1.0)


def procrustes_rotation(M) -> np.ndarray:
    """The orthogonal R that maximises trace(R^T M): R = P Q^T for M = P S Q^T.

    This is the orthogonal Procrustes solution (a textbook result via the
    SVD, np.linalg.svd); it also minimises ||B - X R||_F for M = X^T B.
    """
    P, _, Qt = np.linalg.svd(np.asarray(M, dtype=np.float64))
    return P @ Qt


def itq_loss(X, R) -> float:
    """Quantisation loss ||sign(X R) - X R||_F^2."""
    Y = np.asarray(X, dtype=np.float64) @ np.asarray(R, dtype=np.float64)
    return float(np.sum((sign_pm1(Y) - Y) ** 2))


def joint_itq_rotation(U, V, iters: int = 50, R0=None) -> np.ndarray:
    """Joint-ITQ rotation (s x s) of the stacked factors X = [U; V]."""
    X = np.vstack([np.asarray(U, dtype=np.float64), np.asarray(V, dtype=np.float64)])
    s = X.shape[1]
    R = np.eye(s) if R0 is None else np.asarray(R0, dtype=np.float64).copy()
    for _ in range(int(iters)):
        B = sign_pm1(X @ R)                  # quantise with the current rotation
        R = procrustes_rotation(X.T @ B)     # best rotation for these codes
    return R


def joint_itq(U, V, iters: int = 50, R0=None):
    """(U R, V R, R) with R the Joint-ITQ rotation; (U R)(V R)^T = U V^T."""
    R = joint_itq_rotation(U, V, iters, R0)
    return (np.asarray(U, dtype=np.float64) @ R, np.asarray(V, dtype=np.float64) @ R, R)


# --------------------------------------------------------------------------
# Stack wiring (not on the pages: linear stand-ins for the parts of a
# transformer block that are not LittleBit layers)
# --------------------------------------------------------------------------
def combine(ys, c: float) -> np.ndarray:
    """fp16(c * sum(ys)) computed in float64 from fp16 producer outputs."""
    acc = None
    for y in ys:
        v = _f64(y)
        acc = v if acc is None else acc + v
    return (float(c) * acc).astype(np.float16)


def stack_units(kind: str, n_layers: int) -> list:
    """Unit sizes of a stack: matrices in one unit share one input.

    ``mlp``: per layer [gate, up], [down].  ``block``: per layer
    [q, k, v], [o], [gate, up], [down].  A unit's input is the previous
    unit's outputs summed and scaled by kappa / sqrt(n_prev) (the first
    unit reads the stack input); the stack output is the last unit's
    combine.
    """
    per = {"mlp": [2, 1], "block": [3, 1, 2, 1]}[kind]
    return per * int(n_layers)
