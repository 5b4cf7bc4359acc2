"""Seeded synthetic inputs for the LittleBit linear forward.

This module only draws random numbers.  It holds none of the layer's
arithmetic, so both the float64 oracle and the HIP path can take their
inputs from it without sharing any computation.

Recipe (the pages publish no trained LittleBit checkpoints, so every
tensor is synthetic, with the layer shapes of Llama2-7B / Llama2-70B):

* sign factors S_U (b x s) and S_V (a x s): iid Bernoulli(1/2) bits, one
  bit per entry, drawn as whole uint32 words in the canonical layout
  (row-major, ``ceil(s/32)`` words per row, entry k of a row in bit
  ``k % 32`` of word ``k // 32``; bit 1 means +1, bit 0 means -1).
  Padding bits past ``s`` are zero.
* h (b) and g (a) ~ U[0.5, 1.5], rounded to fp16.
* l (s): ``fp16(u_k / sqrt(a*s))`` with u_k ~ U[0.5, 1.5], computed in
  float64 and rounded once.
* x (M x a) ~ N(0, 1), rounded to fp16.

Streams: every (seed, layer, matrix, path) tuple gets its own PCG64
generator through ``numpy.random.SeedSequence``; activations use the key
(seed, ACT_KEY, stream).  Inside one path the draw order is S_U words,
S_V words, h, g, u.
"""
from __future__ import annotations

import numpy as np

ACT_KEY = 0x5EED_AC7


def words_per_row(s: int) -> int:
    return (int(s) + 31) // 32


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def random_sign_words(rng: np.random.Generator, rows: int, s: int) -> np.ndarray:
    """Uniform random canonical sign words, padding bits cleared."""
    w = words_per_row(s)
    words = rng.integers(0, 1 << 32, size=(rows, w), dtype=np.uint32)
    tail = s % 32
    if tail:
        words[:, -1] &= np.uint32((1 << tail) - 1)
    return words


def path_inputs(a: int, b: int, s: int, seed: int, layer: int = 0, matrix: int = 0,
                path: int = 0) -> dict:
    """One path's (S_U words, S_V words, h, g, l); scales as np.float16."""
    rng = _rng(seed, layer, matrix, path)
    su = random_sign_words(rng, b, s)
    sv = random_sign_words(rng, a, s)
    h = rng.uniform(0.5, 1.5, size=b).astype(np.float16)
    g = rng.uniform(0.5, 1.5, size=a).astype(np.float16)
    u = rng.uniform(0.5, 1.5, size=s)
    l = (u / np.sqrt(float(a) * float(s))).astype(np.float16)
    return {"a": int(a), "b": int(b), "s": int(s), "su": su, "sv": sv, "h": h, "g": g, "l": l}


def layer_inputs(a: int, b: int, s: int, residual: bool, seed: int, layer: int = 0,
                 matrix: int = 0) -> list:
    """All paths of one layer: one dict per path (two when residual)."""
    n = 2 if residual else 1
    return [path_inputs(a, b, s, seed, layer, matrix, p) for p in range(n)]


def activations(M: int, a: int, seed: int, stream: int = 0) -> np.ndarray:
    """x ~ N(0,1) rounded to fp16, shape (M, a)."""
    rng = _rng(seed, ACT_KEY, stream)
    return rng.standard_normal((int(M), int(a))).astype(np.float16)


def garbage_padding(words: np.ndarray, s: int, seed: int) -> np.ndarray:
    """Copy of ``words`` with random bits written into the padding past s."""
    out = words.copy()
    tail = s % 32
    if tail:
        rng = _rng(seed, 0xBAD)
        junk = rng.integers(0, 1 << 32, size=out.shape[0], dtype=np.uint64).astype(np.uint32)
        pad_mask = np.uint32((~((1 << tail) - 1)) & 0xFFFFFFFF)
        out[:, -1] |= junk & pad_mask
    return out


# ---------------------------------------------------------------------------
# Real-valued stand-ins for initialisation from real weights (the pages start
# from pretrained weights, which are not available here).
# ---------------------------------------------------------------------------
FACTOR_KEY = 0xFAC7
WEIGHT_KEY = 0x3E16


def factors(a: int, b: int, s: int, seed: int, stream: int = 0):
    """Real factors U (b x s) and V (a x s), float32, shaped like rank-s SVD factors.

    Columns of a truncated SVD's U sqrt(Sigma) are orthogonal with decaying
    norms; here U = diag(r_U) G_U diag(d) and V = diag(r_V) G_V diag(d) with
    G ~ N(0, 1), d_k = (k + 1) ** -0.25 (a decaying spectrum), and row gains
    r ~ lognormal(0, 0.5) (uneven channel magnitudes).  Random Gaussian
    columns are near-orthogonal for many rows.  Draw order: r_U, G_U, r_V,
    G_V.
    """
    rng = _rng(seed, FACTOR_KEY, stream)
    d = (np.arange(int(s), dtype=np.float64) + 1.0) ** -0.25
    rU = rng.lognormal(0.0, 0.5, int(b))
    U = (rU[:, None] * rng.standard_normal((int(b), int(s)))) * d[None, :]
    rV = rng.lognormal(0.0, 0.5, int(a))
    V = (rV[:, None] * rng.standard_normal((int(a), int(s)))) * d[None, :]
    return U.astype(np.float32), V.astype(np.float32)


def weight_matrix(a: int, b: int, seed: int) -> np.ndarray:
    """A dense stand-in weight W (b x a), float64: row gains x N(0, 1/a) x column gains.

    W = diag(r) G diag(c) / sqrt(a) with r, c ~ lognormal(0, 0.5) and G ~
    N(0, 1): uneven row and column magnitudes, as in trained linear layers.
    Draw order: r, G, c.
    """
    rng = _rng(seed, WEIGHT_KEY)
    r = rng.lognormal(0.0, 0.5, int(b))
    G = rng.standard_normal((int(b), int(a)))
    c = rng.lognormal(0.0, 0.5, int(a))
    return (r[:, None] * G * c[None, :]) / np.sqrt(float(a))


def kappa(paths: int) -> float:
    """Gain that keeps stacked activations O(1) under this recipe.

    With independent random signs, E[y^2] = P * E[h^2] * E[g^2] * E[x^2] *
    a * sum_k E[l_k^2] = P * (13/12)^3 for x ~ N(0,1), since
    E[U(0.5,1.5)^2] = 13/12 and sum_k E[l_k^2] = (13/12) / a.  The stack
    wiring scales each combine by kappa = (P * (13/12)^3) ** -0.5.
    """
    return float((paths * (13.0 / 12.0) ** 3) ** -0.5)


# ---------------------------------------------------------------------------
# Workloads: layer shapes of the measured configurations (Llama2-7B and
# Llama2-70B linear layers at the stated bits per weight).  Pure data.
# ---------------------------------------------------------------------------
WORKLOADS = {
    # name: (seed, M, per-block [(a, b, s, residual)], per-block unit sizes, blocks)
    "tiny_256": (0, 1, [(256, 256, 32, False)], [1], 1),
    "llama7b_attn_proj_4096": (1, 1, [(4096, 4096, 86, True)], [1], 1),
    "llama7b_mlp_stack": (2, 1, [(4096, 11008, 133, True), (4096, 11008, 133, True),
                                 (11008, 4096, 133, True)], [2, 1], 32),
    "llama70b_mlp_stack": (3, 1, [(8192, 28672, 302, True), (8192, 28672, 302, True),
                                  (28672, 8192, 302, True)], [2, 1], 80),
    "llama7b_full_stack_M128": (4, 128, [(4096, 4096, 290, True)] * 4 +
                                [(4096, 11008, 431, True), (4096, 11008, 431, True),
                                 (11008, 4096, 431, True)], [3, 1, 2, 1], 32),
}


def workload(name: str, blocks: int | None = None) -> dict:
    """Shapes, unit sizes, M and seed of a workload (optionally fewer blocks)."""
    seed, M, per, units, nb = WORKLOADS[name]
    nb = nb if blocks is None else int(blocks)
    layers = []
    for blk in range(nb):
        for mi, (a, b, s, res) in enumerate(per):
            layers.append({"a": a, "b": b, "s": s, "residual": res, "block": blk,
                           "matrix": mi, "seed": seed})
    return {"name": name, "seed": seed, "M": M, "layers": layers, "units": list(units) * nb,
            "blocks": nb, "per_block": len(per)}


def workload_layer_inputs(spec: dict) -> list:
    """Paths of one layer of a workload: stream (seed, block, matrix, path)."""
    return layer_inputs(spec["a"], spec["b"], spec["s"], spec["residual"], spec["seed"],
                        spec["block"], spec["matrix"])
