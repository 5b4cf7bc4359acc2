"""Host re-layout of the sign bits, on the CPU, in a sanitizer build.

The library's host functions that turn canonical sign words into the
device layouts (binary_rank_gemv_littlebitlinear_amd/csrc/lb_layout.cpp)
are compiled here together with a small driver (tests/native/) under
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts the
driver), and their output is compared with each layout's definition
evaluated in numpy from the +-1 matrices that ``oracle.unpack_signs`` gives
([LB news] Sec. 2: binarised factors stored as bits).  The read-back
functions must return ``oracle.pack_signs`` of those matrices: the
canonical words with the padding bits cleared.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import lb_synth
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER_SRC = os.path.join(ROOT, "tests", "native", "layout_check.cpp")
LAYOUT_SRC = os.path.join(ROOT, "binary_rank_gemv_littlebitlinear_amd", "csrc", "lb_layout.cpp")
SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    r = subprocess.run([cxx, *SAN_FLAGS, DRIVER_SRC, LAYOUT_SRC, "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return exe


def _run(driver, tmp_path, a, b, s, paths, order=0):
    P = len(paths)
    Wk = (s + 31) // 32
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([a, b, s, P, order], dtype=np.int64).tobytes())
        for p in paths:
            f.write(np.ascontiguousarray(p["su_in"], dtype=np.uint32).tobytes())
            f.write(np.ascontiguousarray(p["sv_in"], dtype=np.uint32).tobytes())
            f.write(np.ascontiguousarray(p["h"], dtype=np.uint16).tobytes())
            f.write(np.ascontiguousarray(p["g"], dtype=np.uint16).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, str(inp), str(out)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=env, timeout=120)
    assert r.returncode == 0, f"sanitized driver failed ({r.returncode}):\n{r.stdout}"
    assert "runtime error" not in r.stdout, r.stdout
    d = _dims(a, b, s, P)
    raw = np.fromfile(out, dtype=np.uint8)
    off = 0

    def take(dtype, n):
        nonlocal off
        nb = np.dtype(dtype).itemsize * n
        v = raw[off:off + nb].view(dtype)
        off += nb
        return v

    res = {
        "sv16": take(np.uint16, d["T16v"] * d["Lp"]).reshape(d["T16v"], d["Lp"]),
        "su2t": take(np.uint32, d["T16b"] * P * Wk * 16).reshape(d["T16b"], P, Wk, 16),
        "sv1m": take(np.uint32, d["R1"] * d["L"]).reshape(d["R1"], d["L"]),
        "su2m": take(np.uint32, P * Wk * d["b16"]).reshape(P, Wk, d["b16"]),
        "ht": take(np.uint16, d["T16b"] * P * 16).reshape(d["T16b"], P, 16),
        "gt": take(np.uint16, d["T16a"] * P * 16).reshape(d["T16a"], P, 16),
        "back": [],
    }
    for _ in range(P):
        su = take(np.uint32, b * Wk).reshape(b, Wk)
        sv = take(np.uint32, a * Wk).reshape(a, Wk)
        res["back"].append((su, sv))
    assert off == raw.size, "driver wrote an unexpected number of bytes"
    return res


def _dims(a, b, s, P):
    L = P * s
    R1 = (a + 31) // 32
    return {"L": L, "Lp": (L + 7) // 8 * 8, "R1": R1, "T16v": 2 * R1, "T16a": (a + 15) // 16,
            "T16b": (b + 15) // 16, "b16": (b + 15) // 16 * 16, "a16": (a + 15) // 16 * 16}


def _words_from_bits(bits, width):
    """bits (..., n * width) of 0/1 -> (..., n) words, bit k of a word = bits[k]."""
    sh = bits.shape[:-1] + (bits.shape[-1] // width, width)
    w = bits.reshape(sh).astype(np.uint64) << np.arange(width, dtype=np.uint64)
    return w.sum(axis=-1)


def _mfma_order(words):
    """The matrix-core bit order: bits inverted, element 8 g + e of the word
    to bit 15 - e/2 - 4 g (e even) or 31 - (e - 1)/2 - 4 g (e odd)."""
    words = np.asarray(words, dtype=np.uint64)
    out = np.zeros_like(words)
    for el in range(32):
        g, e = divmod(el, 8)
        pos = 15 - e // 2 - 4 * g if e % 2 == 0 else 31 - (e - 1) // 2 - 4 * g
        flip = ((words >> np.uint64(el)) & np.uint64(1)) ^ np.uint64(1)
        out |= flip << np.uint64(pos)
    return out.astype(np.uint32)


def _expected(a, b, s, paths):
    P = len(paths)
    d = _dims(a, b, s, P)
    Wk = (s + 31) // 32
    SV = [oracle.unpack_signs(p["sv_in"], s) for p in paths]
    SU = [oracle.unpack_signs(p["su_in"], s) for p in paths]
    # S_V bits by input row and latent column, zero padding
    bv = np.zeros((d["T16v"] * 16, d["Lp"]), dtype=np.uint8)
    for p in range(P):
        bv[:a, p * s:(p + 1) * s] = SV[p] > 0
    sv16 = _words_from_bits(bv.reshape(d["T16v"], 16, d["Lp"]).transpose(0, 2, 1), 16)[..., 0]
    joined = sv16[0::2, :d["L"]] | (sv16[1::2, :d["L"]] << np.uint64(16))
    # S_U words by output row, zero padding
    su2t = np.zeros((d["T16b"], P, Wk, 16), dtype=np.uint64)
    su2m = np.zeros((P, Wk, d["b16"]), dtype=np.uint32)
    for p in range(P):
        bu = np.zeros((d["b16"], Wk * 32), dtype=np.uint8)
        bu[:b, :s] = SU[p] > 0
        w = _words_from_bits(bu, 32)  # b16 x Wk
        su2t[:, p] = w.reshape(d["T16b"], 16, Wk).transpose(0, 2, 1)
        su2m[p] = _mfma_order(w.T)
    ht = np.zeros((d["T16b"], P, 16), dtype=np.uint16)
    gt = np.zeros((d["T16a"], P, 16), dtype=np.uint16)
    for p in range(P):
        hp = np.zeros(d["b16"], dtype=np.uint16)
        hp[:b] = paths[p]["h"]
        gp = np.zeros(d["a16"], dtype=np.uint16)
        gp[:a] = paths[p]["g"]
        ht[:, p] = hp.reshape(-1, 16)
        gt[:, p] = gp.reshape(-1, 16)
    return {"sv16": sv16.astype(np.uint16), "su2t": su2t.astype(np.uint32),
            "sv1m": _mfma_order(joined), "su2m": su2m, "ht": ht, "gt": gt,
            "back": [(oracle.pack_signs(SU[p]), oracle.pack_signs(SV[p])) for p in range(P)]}


def _paths(a, b, s, P, seed, garbage):
    out = []
    for p in range(P):
        q = lb_synth.path_inputs(a, b, s, seed=seed, path=p)
        su, sv = q["su"], q["sv"]
        if garbage:
            su = lb_synth.garbage_padding(su, s, seed=seed + 10 + p)
            sv = lb_synth.garbage_padding(sv, s, seed=seed + 20 + p)
        out.append({"su_in": su, "sv_in": sv, "h": q["h"].view(np.uint16), "g": q["g"].view(np.uint16)})
    return out


SHAPES = [
    (1, 1, 1, 1), (1, 1, 1, 2), (16, 16, 32, 1), (17, 15, 31, 2), (32, 32, 33, 2),
    (37, 45, 33, 2), (40, 200, 1, 1), (64, 48, 64, 1), (100, 17, 95, 2), (513, 300, 70, 2),
    (1024, 768, 130, 2),
]


@pytest.mark.parametrize("a,b,s,P", SHAPES)
def test_layouts_match_their_definitions(driver, tmp_path, a, b, s, P):
    paths = _paths(a, b, s, P, seed=7 * a + b + s, garbage=True)
    got = _run(driver, tmp_path, a, b, s, paths)
    exp = _expected(a, b, s, paths)
    for key in ("sv16", "su2t", "sv1m", "su2m", "ht", "gt"):
        assert np.array_equal(got[key], exp[key]), f"{key} differs at a={a} b={b} s={s} P={P}"
    for p in range(P):
        assert np.array_equal(got["back"][p][0], exp["back"][p][0]), f"S_U read-back, path {p}"
        assert np.array_equal(got["back"][p][1], exp["back"][p][1]), f"S_V read-back, path {p}"


@pytest.mark.parametrize("a,b,s", [(37, 45, 33), (130, 70, 65)])
def test_path_order_does_not_matter(driver, tmp_path, a, b, s):
    """Setting path 1 before path 0 leaves the same layouts: each put
    replaces only its own path's bits."""
    paths = _paths(a, b, s, 2, seed=99, garbage=True)
    fwd = _run(driver, tmp_path, a, b, s, paths, order=0)
    rev = _run(driver, tmp_path, a, b, s, paths, order=1)
    for key in ("sv16", "su2t", "sv1m", "su2m", "ht", "gt"):
        assert np.array_equal(fwd[key], rev[key]), key


def test_mfma_order_gives_the_operand_sign_flips():
    """The matrix-core order's stated purpose, checked on the definition:
    (w << (4 g + j)) & 0x80008000 has bit 15 = the flip (1 = -1) of element
    8 g + 2 j and bit 31 = that of element 8 g + 2 j + 1 of the canonical
    word."""
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2 ** 32, size=64, dtype=np.uint64)
    perm = _mfma_order(words).astype(np.uint64)
    for g in range(4):
        for j in range(4):
            sh = (perm << np.uint64(4 * g + j)) & np.uint64(0xFFFFFFFF)
            lo = (sh >> np.uint64(15)) & np.uint64(1)
            hi = (sh >> np.uint64(31)) & np.uint64(1)
            e0, e1 = 8 * g + 2 * j, 8 * g + 2 * j + 1
            assert np.array_equal(lo, ((words >> np.uint64(e0)) & np.uint64(1)) ^ np.uint64(1))
            assert np.array_equal(hi, ((words >> np.uint64(e1)) & np.uint64(1)) ^ np.uint64(1))


def test_sanitizer_is_active(driver, tmp_path):
    """The build really carries the sanitizers: a header with a negative
    size is refused before any access, and a truncated input file makes the
    driver exit with an error rather than read past its buffers."""
    bad = tmp_path / "bad.bin"
    bad.write_bytes(np.array([4, 4, 4, 1, 0], dtype=np.int64).tobytes())  # no payload
    r = subprocess.run([driver, str(bad), str(tmp_path / "o.bin")], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=60)
    assert r.returncode == 2 and "short read" in r.stdout
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, driver], stdout=subprocess.PIPE, text=True).stdout
        assert "__asan_init" in syms and "__ubsan_handle" in syms
