"""CPU-only checks of the C ABI: the library loads, exports every symbol
the header declares, and its host-side arithmetic (effective bits of the
LittleBit-2 column Ch. 1, rank solve, argument checks) is exact.  No call
here touches a GPU."""
import ctypes
import re
from fractions import Fraction

import pytest

import oracle
from tests import lbtest


def _header_functions():
    text = open(lbtest.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _header_functions()
    for n in ("lb_create", "lb_pack_signs", "lb_set_scales", "lb_forward", "lb_eff_bits",
              "lb_destroy", "lb_stack_create", "lb_stack_forward"):
        assert n in names


def test_library_exports_every_header_symbol():
    lbm = lbtest.ensure_built()
    lib = ctypes.CDLL(lbm.LIB_PATH)
    missing = [n for n in _header_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding exposes the same names
    for n in _header_functions():
        assert hasattr(lbm, n), n
    assert set(lbm.EXPORTED) == set(_header_functions())


CASES = [(256, 256, 32, False), (4096, 4096, 86, True), (4096, 11008, 133, True),
         (11008, 4096, 133, True), (8192, 28672, 302, True), (28672, 8192, 302, True),
         (4096, 4096, 290, True), (4096, 11008, 431, True), (1, 1, 0, False), (3, 5, 7, True)]


@pytest.mark.parametrize("a,b,s,res", CASES)
def test_eff_bits_exact(a, b, s, res):
    lbm = lbtest.ensure_built()
    n, d = lbm.lb_eff_bits(a, b, s, res)
    assert Fraction(n, d) == oracle.eff_bits(a, b, s, res)
    assert n == oracle.num_bits(a, b, s, res) and d == a * b


@pytest.mark.parametrize("a,b", [(4096, 4096), (4096, 11008), (11008, 4096), (8192, 28672),
                                 (28672, 8192), (100, 37), (64, 48)])
@pytest.mark.parametrize("num,den", [(1, 10), (3, 10), (55, 100), (2, 1)])
@pytest.mark.parametrize("res", [False, True])
def test_rank_for_bpw_matches_oracle(a, b, num, den, res):
    lbm = lbtest.ensure_built()
    try:
        want = oracle.rank_for_bpw(a, b, Fraction(num, den), res)
    except ValueError:
        with pytest.raises(lbm.LBError) as ei:
            lbm.lb_rank_for_bpw(a, b, num, den, res)
        assert ei.value.status == lbm.LB_EINVAL
        return
    assert lbm.lb_rank_for_bpw(a, b, num, den, res) == want


def test_host_argument_errors():
    lbm = lbtest.ensure_built()
    lib = lbm.load_library()
    n, d = ctypes.c_uint64(), ctypes.c_uint64()
    assert lib.lb_eff_bits(0, 4, 4, 0, ctypes.byref(n), ctypes.byref(d)) == lbm.LB_EINVAL
    assert lib.lb_eff_bits(4, 4, 4, 2, ctypes.byref(n), ctypes.byref(d)) == lbm.LB_EINVAL
    assert lib.lb_eff_bits(4, 4, 4, 0, None, ctypes.byref(d)) == lbm.LB_EINVAL
    # 64-bit overflow of the numerator is reported, not wrapped
    big = 1 << 40
    assert lib.lb_eff_bits(big, big, big, 1, ctypes.byref(n), ctypes.byref(d)) == lbm.LB_EINVAL
    out = ctypes.c_void_p()
    assert lib.lb_create(0, 4, 4, 0, ctypes.byref(out)) == lbm.LB_EINVAL
    assert lib.lb_create(4, 4, 4, 3, ctypes.byref(out)) == lbm.LB_EINVAL
    assert lib.lb_create(4, 4, 5000, 0, ctypes.byref(out)) == lbm.LB_EINVAL
    assert lib.lb_create(4, 4, 4, 0, None) == lbm.LB_EINVAL
    assert lib.lb_forward(None, None, None, 1, None) == lbm.LB_EINVAL
    assert lib.lb_init_from_factors(None, 0, None, None, None, None) == lbm.LB_EINVAL
    assert lib.lb_joint_itq(None, None, 4, 4, 4, 50, None, None, None) == lbm.LB_EINVAL
    assert lib.lb_joint_itq(8, 8, 4, 4, 5000, 50, None, 8, None) == lbm.LB_EINVAL
    assert lib.lb_joint_itq(8, 8, 4, 4, 4, -1, None, 8, None) == lbm.LB_EINVAL
    assert lib.lb_joint_itq(8, 8, 4, 4, 4, 1, None, 12, None) == lbm.LB_EINVAL
    assert lib.lb_get_scales(None, 0, None, None, None) == lbm.LB_EINVAL
    assert lib.lb_prepare(None, 64) == lbm.LB_EINVAL
    assert lib.lb_layer_device_bytes(None, None, None) == lbm.LB_EINVAL
    assert lib.lb_stack_create(None, 0, None, 0, 1.0, ctypes.byref(out)) == lbm.LB_EINVAL
    assert b"NULL" in lib.lb_last_error() or len(lib.lb_last_error()) > 0
    assert lib.lb_status_str(lbm.LB_ENOTREADY) == b"LB_ENOTREADY"
    assert lib.lb_destroy(None) == lbm.LB_OK
    assert lib.lb_version() >= 100
