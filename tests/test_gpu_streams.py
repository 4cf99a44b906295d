"""Calls on two streams at once, each with its own workspace, give the same
rows as the oracle: the library keeps no state between calls, so calls that
overlap on the device do not interfere (bit-exact, integer inputs)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic as syn

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_tensor(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


@pytest.fixture(scope="module")
def pv():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import top_token_selection_amd as pv
    return pv


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_overlapping_calls_on_two_streams(pv, mode):
    S, H, D, top_k, g, ratio = 3000, 2, 128, 128, 8, 2.0
    print(f"\n[two streams] S={S} H={H} D={D} k={top_k} g={g} {mode}", flush=True)
    sets = []
    for seed in (8101, 8201):
        q = syn.integers((S, H, D), seed, 4, "bf16")
        k = syn.integers((S, H, D), seed + 1, 4, "bf16")
        want, _ = oracle.prefill(q, k, top_k, g, ratio, mode)
        sets.append((dev_tensor(q), dev_tensor(k), want))
    ws_bytes = pv.prefill_workspace_bytes(S, H, D, top_k, g, ratio, mode, torch.bfloat16)
    ws = [torch.empty(ws_bytes, dtype=torch.uint8, device=DEV) for _ in sets]
    outs = [torch.full((S, H, top_k), -7, dtype=torch.int32, device=DEV) for _ in sets]
    streams = [torch.cuda.Stream() for _ in sets]
    torch.cuda.synchronize()
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        # both calls are enqueued before either is waited for
        for (q, k, _), w, o, s in zip(sets, ws, outs, streams):
            with torch.cuda.stream(s):
                pv.index_prefill(q, k, top_k, g, ratio, mode, workspace=w, out=o)
        torch.cuda.synchronize()
        for (_, _, want), o in zip(sets, outs):
            np.testing.assert_array_equal(o.cpu().numpy(), want)
        for o in outs:
            o.fill_(-7)
