"""C-ABI checks that need no GPU: the library loads, exports every function
include/pivot.h declares, and rejects bad arguments on the host with the
documented status codes before anything touches the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pivot.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"extern", "sizeof", "if", "defined"}
    return sorted({n for n in names if n not in skip})


@pytest.fixture(scope="module")
def pv():
    import top_token_selection_amd as pv
    return pv


def test_header_declares_the_abi():
    fns = declared_functions()
    for name in ("pivot_index_prefill", "pivot_index_decode", "dense_index"):
        assert name in fns


def test_library_exports_every_declared_symbol(pv):
    lib = ctypes.CDLL(pv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(pv.EXPORTED)


def test_status_strings(pv):
    for code in (0, -1, -2, -3, -4):
        assert pv.lib.pivot_status_string(code)
    assert pv.lib.pivot_status_string(12345) == b"unknown status"


@pytest.mark.parametrize("top_k,ratio,K", [(64, 2.0, 128), (2048, 2.0, 4096), (3, 1.5, 4),
                                           (3, 1.1, 3), (10, 2.55, 25), (5, 1.0, 5)])
def test_candidate_count_closed_form(pv, top_k, ratio, K):
    """K = int(top_k * candidate_ratio) ("Show Me The Code")."""
    assert pv.candidate_count(top_k, ratio) == K


@pytest.mark.parametrize("top_k,ratio", [(5, 0.9), (0, 2.0), (4, float("nan")), (4, -1.0), (4, float("inf"))])
def test_candidate_count_rejects(pv, top_k, ratio):
    K = ctypes.c_int64(-7)
    assert pv.lib.pivot_candidate_count(top_k, ratio, ctypes.byref(K)) == pv.PIVOT_EINVAL
    assert K.value == -7


def test_workspace_sizes(pv):
    f = pv.lib.pivot_prefill_workspace_bytes
    full = f(65536, 64, 128, 2048, 8, 2.0, 0, 1)
    one = f(65536, 1, 128, 2048, 8, 2.0, 0, 1)
    assert 0 < one < full
    # bytes grow linearly with heads on top of a fixed part
    two = f(65536, 2, 128, 2048, 8, 2.0, 0, 1)
    assert full - one == 63 * (two - one)
    assert f(0, 1, 128, 64, 8, 2.0, 0, 1) == 0        # S < 1
    assert f(64, 1, 96, 8, 8, 2.0, 0, 1) == 0         # D unsupported
    assert f(64, 1, 64, 8, 8, 2.0, 3, 1) == 0         # bad mode
    # the literal per-position Refine scans one row per position: its
    # workspace grows like g = 1 Refine's, not like one row per group
    assert f(4096, 1, 128, 64, 8, 2.0, 2, 1) > f(4096, 1, 128, 64, 8, 2.0, 0, 1)
    assert f(64, 1, 64, 8193, 8, 1.0, 0, 1) == 0      # top_k above 8192
    assert f(64, 1, 64, 4096, 8, 2.5, 0, 1) == 0      # K above 8192
    # K up to 8192 is accepted; beyond 4096 candidates Refine adds the
    # global score rows of its row select to the workspace
    assert f(64, 1, 64, 2048, 8, 4.0, 0, 1) > f(64, 1, 64, 2048, 8, 2.0, 0, 1) > 0
    assert f(64, 1, 64, 8192, 8, 1.0, 1, 1) > 0
    assert pv.lib.dense_index_workspace_bytes(1024, 8, 64, 64, 0) > 0
    # the scan's key tiles span 32 sampled rows through 32-bit offsets: at
    # S = 2^31 - 2 the sampling stride (2^20 keys) of 128-byte rows passes
    # 4 GiB and the call is refused; at S = 2^28 (stride 2^17) it is not
    assert f((1 << 31) - 2, 1, 64, 64, 8, 2.0, 0, 1) == 0
    assert f(1 << 28, 1, 64, 64, 8, 2.0, 0, 1) > 0
    ctx = (ctypes.c_int64 * 3)(5, 9, 100)
    assert pv.lib.pivot_decode_workspace_bytes(3, ctx, 2, 8, 128, 64, 2.0, 0, 1) > 0
    bad = (ctypes.c_int64 * 2)(5, 0)
    assert pv.lib.pivot_decode_workspace_bytes(2, bad, 2, 8, 128, 64, 2.0, 0, 1) == 0


def _prefill(pv, **kw):
    a = dict(q=256, k=256, dtype=1, S=64, H=2, D=64, top_k=8, g=8, ratio=2.0, mode=0,
             out=256, sc=None, ws=256, wsb=1 << 40, st=None)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return pv.lib.pivot_index_prefill(vp(a["q"]), vp(a["k"]), a["dtype"], a["S"], a["H"], a["D"],
                                      a["top_k"], a["g"], a["ratio"], a["mode"], vp(a["out"]),
                                      vp(a["sc"]), vp(a["ws"]), a["wsb"], vp(a["st"]))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(out=None), -1),
    (dict(S=0), -1), (dict(H=0), -1), (dict(g=0), -1), (dict(top_k=0), -1),
    (dict(dtype=7), -1), (dict(mode=3), -1), (dict(ratio=0.5), -1),
    (dict(D=96), -2), (dict(top_k=8193, ratio=1.0), -2), (dict(top_k=8192, ratio=1.5), -2),
    (dict(top_k=4096, ratio=2.001), -2),
    (dict(ws=None), -3), (dict(wsb=16), -3),
    (dict(q=264), -1), (dict(k=258), -1), (dict(out=258), -1), (dict(sc=257), -1), (dict(ws=264), -3),
])
def test_prefill_validation_before_any_device_work(pv, kw, code):
    # pointers here are fake: an argument error must be found on the host
    assert _prefill(pv, **kw) == code


def test_decode_validation(pv):
    vp = lambda x: ctypes.c_void_p(x)
    A = 256  # a fake, 16-byte aligned address: argument errors are found on the host
    ctx = (ctypes.c_int64 * 2)(10, 20)
    zero = (ctypes.c_int64 * 2)(10, 0)
    L = pv.lib.pivot_index_decode
    assert L(vp(A), vp(A), 1, zero, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, None, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(None, vp(A), 1, ctx, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, ctx, 2, 0, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, ctx, 2, 2, 8, 80, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -2
    assert L(vp(A), vp(A), 1, ctx, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 8, None) == -3
    assert L(vp(A + 8), vp(A), 1, ctx, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A + 2), 1, ctx, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, ctx, 2, 2, 8, 128, 8, 2.0, 0, vp(A), None, vp(A + 4), 1 << 40, None) == -3


def test_dense_validation(pv):
    vp = ctypes.c_void_p
    A = 256
    L = pv.lib.dense_index
    assert L(None, vp(A), 1, 64, 2, 64, 8, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, 64, 2, 64, 0, vp(A), None, vp(A), 1 << 40, None) == -1
    assert L(vp(A), vp(A), 1, 64, 2, 128, 8193, vp(A), None, vp(A), 1 << 40, None) == -2
    assert L(vp(A), vp(A), 1, 64, 2, 64, 8, vp(A), None, None, 0, None) == -3
    assert L(vp(A + 4), vp(A), 1, 64, 2, 64, 8, vp(A), None, vp(A), 1 << 40, None) == -1


def test_sparse_attention_validation(pv):
    vp = ctypes.c_void_p
    A = 256
    L = pv.lib.pivot_sparse_attention
    ok = dict(q=A, k=A, v=A, dtype=1, S=64, H=2, D=64, idx=A, top_k=8, scale=0.125, out=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        p = lambda x: None if x is None else vp(x)
        return L(p(a["q"]), p(a["k"]), p(a["v"]), a["dtype"], a["S"], a["H"], a["D"], p(a["idx"]),
                 a["top_k"], a["scale"], p(a["out"]), None)

    assert call(q=None) == -1
    assert call(idx=None) == -1
    assert call(v=A + 8) == -1
    assert call(out=A + 2) == -1
    assert call(S=0) == -1
    assert call(top_k=0) == -1
    assert call(scale=float("nan")) == -1
    assert call(dtype=5) == -1
    assert call(D=96) == -2
