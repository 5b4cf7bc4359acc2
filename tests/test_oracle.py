"""Pins of the float64 oracle against things other than itself.

Each test checks the oracle against a brute-force loop, a hand-worked
fixture, a closed form, an invariant or a number printed on the pages.
The sources are the LittleBit-2 column (physicalainews.jp, Ch. 1: the
effective-bit count) and the Samsung LittleBit news page (aifrontier.co.jp,
Sec. 1 model-size table, Sec. 2 layer structure).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import lb_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bit(words, r, k):
    """Independent bit reader: plain Python ints, no numpy broadcasting."""
    return (int(words[r][k // 32]) >> (k % 32)) & 1


def _brute_force(x, paths):
    """Dense W by nested loops, then y = x W^T; all in Python floats."""
    a, b, s = paths[0]["a"], paths[0]["b"], paths[0]["s"]
    W = [[0.0] * a for _ in range(b)]
    for p in paths:
        h = [float(v) for v in p["h"]]
        g = [float(v) for v in p["g"]]
        l = [float(v) for v in p["l"]]
        for j in range(b):
            for i in range(a):
                acc = 0.0
                for k in range(s):
                    su = 1.0 if _bit(p["su"], j, k) else -1.0
                    sv = 1.0 if _bit(p["sv"], i, k) else -1.0
                    acc += su * l[k] * sv
                W[j][i] += h[j] * acc * g[i]
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    y = np.zeros((x.shape[0], b))
    for m in range(x.shape[0]):
        for j in range(b):
            y[m, j] = sum(W[j][i] * x[m, i] for i in range(a))
    return y, np.array(W)


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- bit count
@pytest.mark.parametrize("a,b,s,res", [(256, 256, 32, False), (100, 37, 5, True),
                                       (4096, 4096, 86, True), (64, 48, 33, False)])
def test_num_bits_counts_the_stored_tensors(a, b, s, res):
    """The bit count equals what a generated layer actually stores:
    one bit per sign entry plus 16 bits per fp16 scale, summed over paths."""
    paths = lb_synth.layer_inputs(a, b, s, res, seed=3)
    stored = 0
    for p in paths:
        stored += oracle.unpack_signs(p["su"], s).size + oracle.unpack_signs(p["sv"], s).size
        stored += 16 * (p["h"].size + p["g"].size + p["l"].size)
    assert oracle.num_bits(a, b, s, res) == stored
    assert oracle.eff_bits(a, b, s, res) == Fraction(stored, a * b)


def test_workload_ranks_and_floor_property():
    gold = _load("workload_ranks.json")
    for c in gold["cases"]:
        bpw = Fraction(c["bpw"])
        s = oracle.rank_for_bpw(c["a"], c["b"], bpw, c["residual"])
        assert s == c["s"], c
        assert oracle.eff_bits(c["a"], c["b"], s, c["residual"]) <= bpw
        assert oracle.eff_bits(c["a"], c["b"], s + 1, c["residual"]) > bpw
    t = gold["tiny"]
    assert oracle.eff_bits(t["a"], t["b"], t["s"], t["residual"]) == Fraction(t["eff_bits"])


@pytest.mark.parametrize("a,b", [(16, 24), (40, 9), (64, 64)])
@pytest.mark.parametrize("res", [False, True])
def test_rank_solver_matches_linear_search(a, b, res):
    for bpw in (Fraction(1, 2), Fraction(3, 1), Fraction(7, 3)):
        try:
            s = oracle.rank_for_bpw(a, b, bpw, res)
        except ValueError:
            assert oracle.eff_bits(a, b, 0, res) > bpw
            continue
        best = max(k for k in range(0, 4 * (a + b)) if oracle.eff_bits(a, b, k, res) <= bpw)
        assert s == best


def test_model_sizes_printed_on_the_news_page():
    """Loose: residual LittleBit linears + FP16 embeddings/lm_head/norms
    reproduce the printed model sizes within 6%."""
    gold = _load("model_sizes.json")
    for m in gold["models"]:
        d, f, L, kv, V = m["hidden"], m["inter"], m["layers"], m["kv"], m["vocab"]
        bpw = Fraction(m["bpw"])
        shapes = [(d, d), (d, kv), (d, kv), (d, d), (d, f), (d, f), (f, d)]
        bits = 0
        for a, b in shapes:
            s = oracle.rank_for_bpw(a, b, bpw, True)
            bits += oracle.num_bits(a, b, s, True)
        total = L * bits / 8 + 2 * V * d * 2 + (2 * L + 1) * d * 2
        assert abs(total / 1e9 - m["gb"]) / m["gb"] < gold["tolerance"], (m["name"], total / 1e9)


# ---------------------------------------------------------------- packing
def test_pack_hand_example():
    gold = _load("pack_example.json")
    s = gold["s"]
    S = -np.ones((1, s), dtype=np.int8)
    S[0, gold["plus_positions"]] = 1
    assert oracle.pack_signs(S).tolist() == [gold["words"]]
    assert (oracle.unpack_signs(np.array([gold["words"]], dtype=np.uint32), s) == S).all()


@pytest.mark.parametrize("s", [1, 5, 31, 32, 33, 63, 64, 65, 86, 302])
def test_pack_roundtrip_and_padding_ignored(s):
    rng = np.random.default_rng(s)
    S = np.where(rng.random((7, s)) < 0.5, 1, -1).astype(np.int8)
    words = oracle.pack_signs(S)
    assert words.shape == (7, (s + 31) // 32)
    assert (oracle.unpack_signs(words, s) == S).all()
    junk = lb_synth.garbage_padding(words, s, seed=s)
    assert (oracle.unpack_signs(junk, s) == S).all()
    # independent reader agrees bit by bit
    for r in range(7):
        for k in range(s):
            assert (S[r, k] == 1) == bool(_bit(words, r, k))
    # padding of a packed word is zero
    if s % 32:
        assert (words[:, -1] >> np.uint32(s % 32) == 0).all()


def test_sign_count_matches_bits():
    """Count of unpacked sign entries equals the sign part of the bit count."""
    a, b, s = 40, 24, 13
    paths = lb_synth.layer_inputs(a, b, s, True, seed=1)
    n = sum(oracle.unpack_signs(p["su"], s).size + oracle.unpack_signs(p["sv"], s).size for p in paths)
    assert n == 2 * s * (a + b)


# ---------------------------------------------------------------- forward
def test_hand_worked_example():
    gold = _load("hand_forward.json")
    paths = []
    for p in gold["paths"]:
        paths.append({"a": gold["a"], "b": gold["b"], "s": gold["s"],
                      "su": np.array(p["su_words"], dtype=np.uint32),
                      "sv": np.array(p["sv_words"], dtype=np.uint32),
                      "h": np.array(p["h"], np.float16), "g": np.array(p["g"], np.float16),
                      "l": np.array(p["l"], np.float16)})
    x = np.array(gold["x"], dtype=np.float16)
    assert np.array_equal(oracle.forward(x, paths[:1]), np.array(gold["y_path0_only"], float))
    assert np.array_equal(oracle.forward(x, paths), np.array(gold["y_residual"], float))


@pytest.mark.parametrize("a,b,s,res,M", [(5, 3, 2, False, 1), (7, 4, 33, True, 2),
                                         (6, 9, 1, True, 3), (12, 5, 64, False, 2),
                                         (3, 11, 65, True, 1)])
def test_factorized_equals_brute_force_dense(a, b, s, res, M):
    paths = lb_synth.layer_inputs(a, b, s, res, seed=a * 100 + b)
    x = lb_synth.activations(M, a, seed=a + b)
    y_bf, W_bf = _brute_force(x, paths)
    y = oracle.forward(x, paths)
    assert _rel(y, y_bf) <= 1e-12
    assert _rel(oracle.dense_weight(paths), W_bf) <= 1e-12


def _brute_force_latent(x, paths):
    """w[m][p*s + k] = l_k * sum_i S_V[i, k] g_i x[m, i] by loops over Python floats."""
    s = paths[0]["s"]
    a = paths[0]["a"]
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    out = np.zeros((x.shape[0], len(paths) * s))
    for pi, p in enumerate(paths):
        g = [float(v) for v in p["g"]]
        l = [float(v) for v in p["l"]]
        for m in range(x.shape[0]):
            for k in range(s):
                acc = 0.0
                for i in range(a):
                    sv = 1.0 if _bit(p["sv"], i, k) else -1.0
                    acc += sv * g[i] * x[m, i]
                out[m, pi * s + k] = l[k] * acc
    return out


def _brute_force_from_latent(w, paths):
    """y[m][j] = sum_p h_j sum_k S_U[j, k] w[m][p*s + k] by loops over Python floats."""
    s, b = paths[0]["s"], paths[0]["b"]
    y = np.zeros((w.shape[0], b))
    for pi, p in enumerate(paths):
        h = [float(v) for v in p["h"]]
        for m in range(w.shape[0]):
            for j in range(b):
                acc = 0.0
                for k in range(s):
                    su = 1.0 if _bit(p["su"], j, k) else -1.0
                    acc += su * float(w[m, pi * s + k])
                y[m, j] += h[j] * acc
    return y


@pytest.mark.parametrize("a,b,s,res,M", [(5, 3, 2, False, 1), (7, 4, 33, True, 2),
                                         (6, 9, 1, True, 3), (12, 5, 64, False, 2),
                                         (40, 3, 65, True, 1)])
def test_latent_and_second_half_against_loops(a, b, s, res, M):
    """The split halves of the forward (the latent a cache would hold, and the
    product from it) against nested loops, and their composition against the
    brute-force dense forward."""
    paths = lb_synth.layer_inputs(a, b, s, res, seed=a * 31 + s)
    x = lb_synth.activations(M, a, seed=b + s)
    w = oracle.latent(x, paths)
    assert w.shape == (M, len(paths) * s)
    assert _rel(w, _brute_force_latent(x, paths)) <= 1e-12
    assert _rel(oracle.from_latent(w, paths), _brute_force_from_latent(w, paths)) <= 1e-12
    y_bf, _ = _brute_force(x, paths)
    assert _rel(oracle.from_latent(w, paths), y_bf) <= 1e-12


def test_latent_path_order_and_scale():
    """Path 1's columns follow path 0's, and the latent scale l multiplies its
    own column only: doubling l_k of path 1 doubles column s + k alone."""
    a, b, s = 9, 4, 5
    paths = lb_synth.layer_inputs(a, b, s, True, seed=3)
    x = lb_synth.activations(2, a, seed=4)
    w = oracle.latent(x, paths)
    assert np.array_equal(w[:, :s], oracle.latent(x, paths[:1]))
    assert np.array_equal(w[:, s:], oracle.latent(x, paths[1:]))
    p1 = dict(paths[1])
    p1["l"] = p1["l"].copy()
    p1["l"][2] = p1["l"][2] * np.float16(2)
    w2 = oracle.latent(x, [paths[0], p1])
    d = np.zeros_like(w, dtype=bool)
    d[:, s + 2] = True
    assert np.array_equal(w2[~d], w[~d])
    assert np.array_equal(w2[:, s + 2], 2 * w[:, s + 2])


def test_tiny_workload_dense_check():
    """The 256x256, s=32 single-path case against the dense reconstruction."""
    paths = lb_synth.layer_inputs(256, 256, 32, False, seed=0)
    x = lb_synth.activations(1, 256, seed=0)
    W = oracle.dense_weight(paths)
    y_dense = x.astype(np.float64) @ W.T
    assert _rel(oracle.forward(x, paths), y_dense) <= 1e-12


def test_all_plus_signs_is_rank_one():
    a, b, s = 20, 12, 7
    p = lb_synth.path_inputs(a, b, s, seed=5)
    ones = (1 << s) - 1
    p["su"] = np.full((b, 1), ones, np.uint32)
    p["sv"] = np.full((a, 1), ones, np.uint32)
    x = lb_synth.activations(2, a, seed=9)
    f = lambda v: np.asarray(v, np.float64)
    expect = f(p["h"])[None, :] * f(p["l"]).sum() * (x.astype(np.float64) @ f(p["g"]))[:, None]
    assert _rel(oracle.forward(x, [p]), expect) <= 1e-13


def test_unit_vector_returns_column():
    a, b, s = 9, 6, 4
    paths = lb_synth.layer_inputs(a, b, s, True, seed=8)
    _, W = _brute_force(np.zeros((1, a), np.float16), paths)
    for i in range(a):
        e = np.zeros((1, a), np.float16)
        e[0, i] = 1
        assert _rel(oracle.forward(e, paths)[0], W[:, i]) <= 1e-13


def test_zero_input_gives_exact_zero():
    paths = lb_synth.layer_inputs(33, 17, 5, True, seed=2)
    y = oracle.forward(np.zeros((3, 33), np.float16), paths)
    assert (y == 0).all()


def test_rank_one_closed_form():
    """s = 1: y = h * su * l * (sv . (g * x)) for each path."""
    a, b = 11, 7
    p = lb_synth.path_inputs(a, b, 1, seed=4)
    x = lb_synth.activations(1, a, seed=1).astype(np.float64)[0]
    su = np.array([1.0 if _bit(p["su"], j, 0) else -1.0 for j in range(b)])
    sv = np.array([1.0 if _bit(p["sv"], i, 0) else -1.0 for i in range(a)])
    t = sum(sv[i] * float(p["g"][i]) * x[i] for i in range(a))
    expect = np.array([float(p["h"][j]) * su[j] * float(p["l"][0]) * t for j in range(b)])
    assert _rel(oracle.forward(x[None, :].astype(np.float16), [p])[0], expect) <= 1e-13


def _perm_latent(p, perm):
    s = p["s"]
    q = dict(p)
    q["su"] = oracle.pack_signs(oracle.unpack_signs(p["su"], s)[:, perm])
    q["sv"] = oracle.pack_signs(oracle.unpack_signs(p["sv"], s)[:, perm])
    q["l"] = p["l"][perm]
    return q


def test_latent_permutation_invariance():
    a, b, s = 30, 20, 37
    p = lb_synth.path_inputs(a, b, s, seed=6)
    x = lb_synth.activations(2, a, seed=6)
    perm = np.random.default_rng(0).permutation(s)
    assert _rel(oracle.forward(x, [_perm_latent(p, perm)]), oracle.forward(x, [p])) <= 1e-13


def test_sign_flip_invariances():
    a, b, s = 25, 14, 9
    p = lb_synth.path_inputs(a, b, s, seed=7)
    x = lb_synth.activations(2, a, seed=7)
    y = oracle.forward(x, [p])
    k = 4
    SU = oracle.unpack_signs(p["su"], s)
    SV = oracle.unpack_signs(p["sv"], s)
    both = dict(p)
    SU2, SV2 = SU.copy(), SV.copy()
    SU2[:, k] *= -1
    SV2[:, k] *= -1
    both["su"], both["sv"] = oracle.pack_signs(SU2), oracle.pack_signs(SV2)
    assert _rel(oracle.forward(x, [both]), y) <= 1e-13
    # flipping S_V's column only equals negating l_k
    only = dict(p)
    only["sv"] = oracle.pack_signs(SV2)
    neg = dict(p)
    neg["l"] = p["l"].copy()
    neg["l"][k] = -neg["l"][k]
    assert _rel(oracle.forward(x, [only]), oracle.forward(x, [neg])) <= 1e-13


def test_linearity_in_x():
    """f(x1 + 3 x2) = f(x1) + 3 f(x2) on small-integer inputs (exact in fp16)."""
    a, b, s = 40, 16, 12
    paths = lb_synth.layer_inputs(a, b, s, True, seed=10)
    rng = np.random.default_rng(10)
    x1 = rng.integers(-8, 9, size=(2, a)).astype(np.float16)
    x2 = rng.integers(-8, 9, size=(2, a)).astype(np.float16)
    xs = (x1.astype(np.float64) + 3 * x2.astype(np.float64)).astype(np.float16)
    lhs = oracle.forward(xs, paths)
    rhs = oracle.forward(x1, paths) + 3 * oracle.forward(x2, paths)
    assert _rel(lhs, rhs) <= 1e-13


def test_residual_is_sum_of_single_paths():
    a, b, s = 50, 30, 17
    paths = lb_synth.layer_inputs(a, b, s, True, seed=11)
    x = lb_synth.activations(3, a, seed=11)
    y = oracle.forward(x, paths)
    assert _rel(y, oracle.forward(x, paths[:1]) + oracle.forward(x, paths[1:])) <= 1e-14


@pytest.mark.parametrize("which", ["h", "g", "l"])
def test_power_of_two_scaling_exact(which):
    a, b, s = 64, 32, 20
    p = lb_synth.path_inputs(a, b, s, seed=12)
    x = lb_synth.activations(2, a, seed=12)
    q = dict(p)
    q[which] = (p[which].astype(np.float64) * 4).astype(np.float16)
    assert np.array_equal(oracle.forward(x, [q]), 4 * oracle.forward(x, [p]))


@pytest.mark.parametrize("res,expect", [(False, 1.128), (True, 1.595)])
def test_output_rms_statistic(res, expect):
    """rms(y) ~ sqrt(P (13/12)^3) under the synthetic recipe (a dropped or
    doubled scale moves it far outside 10%)."""
    a, b, s = 2048, 512, 64
    paths = lb_synth.layer_inputs(a, b, s, res, seed=21)
    x = lb_synth.activations(8, a, seed=21)
    rms = math.sqrt(float(np.mean(oracle.forward(x, paths) ** 2)))
    assert abs(rms - expect) / expect < 0.10
    assert abs(expect - math.sqrt((2 if res else 1) * (13 / 12) ** 3)) < 1e-3


def test_combine_rounding():
    y1 = np.array([1.0, -2.0, 65504.0], np.float16)
    y2 = np.array([0.5, 2.0, 0.0], np.float16)
    out = oracle.combine([y1, y2], 0.5)
    assert out.dtype == np.float16
    assert out.tolist() == [0.75, 0.0, 32752.0]


def test_stack_units():
    assert oracle.stack_units("mlp", 2) == [2, 1, 2, 1]
    assert oracle.stack_units("block", 1) == [3, 1, 2, 1]


def test_generator_determinism():
    p1 = lb_synth.path_inputs(300, 200, 45, seed=1, layer=2, matrix=1, path=1)
    p2 = lb_synth.path_inputs(300, 200, 45, seed=1, layer=2, matrix=1, path=1)
    p3 = lb_synth.path_inputs(300, 200, 45, seed=1, layer=2, matrix=1, path=0)
    for k in ("su", "sv", "h", "g", "l"):
        assert np.array_equal(p1[k], p2[k])
    assert not np.array_equal(p1["su"], p3["su"])
    # padding bits are zero and scales are in range
    assert (p1["su"][:, -1] >> np.uint32(45 % 32) == 0).all()
    assert p1["h"].min() >= 0.5 and p1["h"].max() <= 1.5
