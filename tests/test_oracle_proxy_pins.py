"""Pins of the oracle's proxy rounding on inputs where the order and the
precision of the sum matter.

The proxy is the mean of the group ("PIVOT Explained", "How It Works"); its
rounding follows the reading used throughout: a float32 sum of the members
in ascending position, one IEEE float32 division by the member count, then
round-to-nearest-even to bf16 for bf16 inputs. Integer inputs of small
magnitude make every summation order exact, so the cases below use members
2^24 apart, where float32 addition rounds. Every expected value is derived
by hand in the docstrings. A mutation check builds copies of the oracle
source with the sum in double, in reverse order, or the division replaced
by a reciprocal multiply, and requires each copy to fail one of these pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

BIG = 2.0 ** 24

# Members of one group of g = 8 in four dimensions (positions in ascending
# order). Derivations, float32 round-to-nearest-even (ulp 2 in [2^24, 2^25)):
#  d0  [2^24, 1, 1, 1, 1, 1, 1, -2^24]
#      2^24 + 1 is halfway between 2^24 and 2^24 + 2; the even significand is
#      2^24, so the running sum stays 2^24 for all six ones; adding -2^24
#      gives 0. Proxy 0 / 8 = 0. (Exact or double sum: 6 -> 0.75; reverse
#      order: -2^24 + 1 = -16777215 is exact, five more ones give -16777210,
#      then + 2^24 = 6 -> 0.75.)
#  d1  [2^24, 3, 0, 0, 0, 0, 0, -2^24]
#      2^24 + 3 = 16777219 lies halfway between 16777218 (significand
#      8388609, odd) and 16777220 (8388610, even): it rounds up to 16777220;
#      then -2^24 leaves 4. Proxy 4 / 8 = 0.5. (Exact: 3 / 8 = 0.375.)
#  d2  [1, 1, 1, 1, 1, 1, 2^24, -2^24]
#      6 + 2^24 = 16777222 is even, exact; the sum ends at 6. Proxy 0.75 in
#      every order.
#  d3  [-2^24, 1, 1, 1, 1, 1, 1, 2^24]
#      the mirror of d0: -16777215 ... -16777210 exactly, then + 2^24 = 6.
#      Proxy 0.75 ascending; in reverse order 2^24 + 1 rounds back to 2^24
#      six times and the sum ends at 0.
# 0, 0.5, 0.75 and 0.375 are bf16 values, so bf16 inputs give the same
# proxies (the members themselves are powers of two, 3 and 0: exact in bf16).
SUM_MEMBERS = np.array([
    [BIG, 1, 1, 1, 1, 1, 1, -BIG],
    [BIG, 3, 0, 0, 0, 0, 0, -BIG],
    [1, 1, 1, 1, 1, 1, BIG, -BIG],
    [-BIG, 1, 1, 1, 1, 1, 1, BIG],
], np.float64).T                      # (8 positions, 4 dims)
SUM_PROXY = np.array([0.0, 0.5, 0.75, 0.75], np.float32)

# m = 3 members [5, 0, 0]: one float32 division 5 / 3 = 1.6666...; in units
# of 2^-23 that is 13981013.33, which rounds to 13981013: bits 0x3FD55555.
# A reciprocal multiply 5 * fl(1/3) (fl(1/3) = 11184811 * 2^-25) gives
# 55924055 * 2^-25 = 13981013.75 * 2^-23, which rounds to 0x3FD55556.
DIV_BITS = 0x3FD55555


def _group(members: np.ndarray, dtype: str):
    """q of shape (m, 1, D) holding the members (exact in either dtype)."""
    q = members[:, None, :].astype(np.float32)
    if dtype == "bf16":
        u = q.view(np.uint32)
        assert ((u & np.uint32(0xFFFF)) == 0).all(), "members must be bf16 values"
        return (u >> np.uint32(16)).astype(np.uint16)
    return q


def _proxy_fn(lib_path=None):
    if lib_path is None:
        return lambda q, g: oracle.proxy(q, g, 0, 0)
    lib = ctypes.CDLL(lib_path)
    vp, i32, i64, ci = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    lib.oracle_proxy.argtypes = [vp, ci, i64, i32, i32, i32, i32, i64, vp]
    lib.oracle_proxy.restype = ci

    def fn(q, g):
        q = np.ascontiguousarray(q)
        out = np.empty(q.shape[2], np.float32)
        dt = 1 if q.dtype == np.uint16 else 0
        assert lib.oracle_proxy(q.ctypes.data_as(vp), dt, q.shape[0], q.shape[1], q.shape[2], g, 0, 0,
                                out.ctypes.data_as(vp)) == 0
        return out
    return fn


def _pins_hold(proxy) -> bool:
    ok = True
    for dtype in ("f32", "bf16"):
        ok &= np.array_equal(proxy(_group(SUM_MEMBERS, dtype), 8), SUM_PROXY)
    p = proxy(_group(np.array([[5.0], [0.0], [0.0]]), "f32"), 3)
    ok &= int(p.view(np.uint32)[0]) == DIV_BITS
    return bool(ok)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_proxy_sums_in_float32_in_position_order(dtype):
    got = oracle.proxy(_group(SUM_MEMBERS, dtype), 8, 0, 0)
    np.testing.assert_array_equal(got, SUM_PROXY)


def test_proxy_divides_once_in_float32():
    got = oracle.proxy(_group(np.array([[5.0], [0.0], [0.0]]), "f32"), 3, 0, 0)
    assert int(got.view(np.uint32)[0]) == DIV_BITS
    # bf16: 1.66666663 rounds to the nearest bf16, 213 / 128 = 1.6640625
    got = oracle.proxy(_group(np.array([[5.0], [0.0], [0.0]]), "bf16"), 3, 0, 0)
    assert float(got[0]) == 213.0 / 128.0


def test_proxy_of_a_ragged_last_group():
    """S = 11, g = 8: group 1 holds positions 8, 9, 10 (m = 3); its proxy is
    5 / 3 in float32 as above, and group 0's is the d0 sum pattern."""
    q = np.zeros((11, 1, 1), np.float32)
    q[:8, 0, 0] = SUM_MEMBERS[:, 0]
    q[8, 0, 0] = 5.0
    assert float(oracle.proxy(q, 8, 0, 0)[0]) == 0.0
    assert int(oracle.proxy(q, 8, 0, 1).view(np.uint32)[0]) == DIV_BITS


MUTATIONS = {
    "double accumulation": [
        ("        float sum = 0.0f;\n", "        double sum = 0.0;\n"),
        ("        float v = sum / (float)m;\n", "        float v = (float)(sum / (double)m);\n"),
    ],
    "reverse order": [
        ("        for (int64_t i = i0; i < i0 + m; ++i)\n            sum += load_elem",
         "        for (int64_t i = i0 + m - 1; i >= i0; --i)\n            sum += load_elem"),
    ],
    "reciprocal multiply": [
        ("        float v = sum / (float)m;\n", "        float v = sum * (1.0f / (float)m);\n"),
    ],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_other_summation_rules(tmp_path, name):
    """Each mutated copy of the oracle's group_proxy fails the pins above
    (the copies live in a temporary directory; the oracle is untouched)."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "pivot_oracle.c")).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so),
                           str(c), "-lm"])
    assert _pins_hold(_proxy_fn()), "the oracle itself must hold the pins"
    assert not _pins_hold(_proxy_fn(str(so))), f"a {name} proxy passes the pins"
