"""pivot_index_decode_noalloc (the decode entry point that allocates
nothing: its scratch is the library's static device array) through the C
ABI against pivot_index_decode with a caller workspace: identical indices
and scores on two calls in a row, the second with a smaller input, and the
host-side rejection of a call whose scratch would exceed the array."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synthetic as syn

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def pv():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import top_token_selection_amd as pv
    return pv


def _inputs(B, H, D, g, lo, hi, seed):
    ctx = syn.decode_lengths(B, lo, hi, seed)
    kc = syn.pareto_keys(int(ctx.sum()), H, D, seed + 1, dtype="bf16")
    q = syn.ar1_queries(B * g, H, D, seed + 2, dtype="bf16")
    dev = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return dev(q), dev(kc), ctx


def _call(pv, fn, q, kc, ctx, g, top_k, ratio, mode, ws=None):
    rows, H, D = q.shape
    out = torch.full((rows, H, top_k), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((rows, H, top_k), 7.0, dtype=torch.float32, device=DEV)
    c = (ctypes.c_int64 * len(ctx))(*[int(x) for x in ctx])
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    m = {"refine": 0, "reuse": 1}[mode]
    if ws is None:
        rc = fn(vp(q), vp(kc), 1, c, len(ctx), g, H, D, top_k, ratio, m, vp(out), vp(sc), st)
    else:
        rc = fn(vp(q), vp(kc), 1, c, len(ctx), g, H, D, top_k, ratio, m, vp(out), vp(sc), vp(ws), ws.numel(), st)
    torch.cuda.synchronize()
    return rc, out, sc


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_noalloc_decode_equals_workspace_decode(pv, mode):
    top_k, ratio = 512, 2.0
    # first a larger step, then a smaller one: the second must not see the
    # first call's leftovers in the shared scratch
    for B, H, g, lo, hi, seed in ((12, 4, 4, 3000, 40000, 31), (3, 2, 2, 700, 5000, 41)):
        print(f"\n[no-alloc decode] {mode} B={B} H={H} g={g} ctx U[{lo}, {hi}]", flush=True)
        q, kc, ctx = _inputs(B, H, 128, g, lo, hi, seed)
        need = pv.decode_workspace_bytes(ctx, g, H, 128, top_k, ratio, mode, torch.bfloat16)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        rc0, want_i, want_s = _call(pv, pv.lib.pivot_index_decode, q, kc, ctx, g, top_k, ratio, mode, ws)
        rc1, got_i, got_s = _call(pv, pv.lib.pivot_index_decode_noalloc, q, kc, ctx, g, top_k, ratio, mode)
        assert rc0 == 0 and rc1 == 0, (rc0, rc1)
        assert torch.equal(got_i, want_i)
        assert torch.equal(got_s, want_s)
        # index-only as well, through the binding
        only = pv.index_decode_noalloc(q, kc, ctx, g, top_k=top_k, candidate_ratio=ratio, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(only, want_i)


def test_noalloc_rejects_a_step_beyond_its_scratch(pv):
    """64 sequences of 131072 keys, H = 8: about 288 MiB of scratch, more
    than the 256 MiB array: refused on the host, outputs untouched."""
    B, g, H, D, top_k = 64, 2, 8, 128, 2048
    ctx = np.full(B, 131072, np.int64)
    need = pv.decode_workspace_bytes(ctx, g, H, D, top_k, 2.0, "refine", torch.bfloat16)
    assert need > (256 << 20)
    out = torch.full((B * g, H, top_k), -7, dtype=torch.int32, device=DEV)
    c = (ctypes.c_int64 * B)(*[int(x) for x in ctx])
    A = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    rc = pv.lib.pivot_index_decode_noalloc(A, A, 1, c, B, g, H, D, top_k, 2.0, 0,
                                           ctypes.c_void_p(out.data_ptr()), None, None)
    torch.cuda.synchronize()
    assert rc == pv.PIVOT_EWORKSPACE
    assert bool((out == -7).all())
