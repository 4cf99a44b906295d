"""GPU parity on seeded random small shapes (integer inputs, bit-exact).

Shapes, group sizes, candidate ratios, top_k and decode context lengths are
drawn from a fixed seed, restricted to the configurations whose float32
scores are all exact (bf16 inputs, or float32 with power-of-two groups that
divide S), so indices, order, padding and scores must equal the oracle's.
"""
from __future__ import annotations

import random

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_tensor(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def draw_cases(seed: int, count: int):
    rng = random.Random(seed)
    cases = []
    while len(cases) < count:
        S = rng.choice([rng.randint(1, 64), rng.randint(65, 700), rng.randint(700, 2000)])
        H = rng.randint(1, 3)
        D = rng.choice([64, 128])
        dtype = rng.choice(["bf16", "bf16", "f32"])
        top_k = rng.choice([1, 2, 3, rng.randint(4, 64), rng.randint(65, 300)])
        g = rng.choice([1, 2, 3, 4, 5, 8, 16, 32])
        ratio = rng.choice([1.0, 1.5, 2.0, 3.0, 4.0])
        if dtype == "f32" and (S % g != 0 or g & (g - 1)):
            continue  # a float32 proxy of such a group is not exact
        cases.append((S, H, D, top_k, g, ratio, dtype, rng.randint(1, 10**6)))
    return cases


CASES = draw_cases(20261203, 24)


@pytest.fixture(scope="module")
def pv():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import top_token_selection_amd as pv
    return pv


@pytest.mark.parametrize("S,H,D,top_k,g,ratio,dtype,seed", CASES)
def test_random_shape_prefill_bit_exact(pv, S, H, D, top_k, g, ratio, dtype, seed):
    print(f"\n[random prefill] S={S} H={H} D={D} k={top_k} g={g} r={ratio} {dtype} seed={seed}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), seed, a, dtype)
    k = syn.integers((S, H, D), seed + 1, a, dtype)
    for mode in ("refine", "reuse"):
        oi, os_ = oracle.prefill(q, k, top_k, g, ratio, mode)
        only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio, mode=mode)
        idx, sc = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio,
                                   mode=mode, return_scores=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(parity.to_host(only), oi)
        np.testing.assert_array_equal(parity.to_host(idx), oi)
        np.testing.assert_array_equal(parity.to_host(sc), os_)
    if S <= 1200:
        oi, os_ = oracle.dense(q, k, top_k)
        idx, sc = pv.dense_index(dev_tensor(q), dev_tensor(k), top_k=top_k, return_scores=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(parity.to_host(idx), oi)
        np.testing.assert_array_equal(parity.to_host(sc), os_)


@pytest.mark.parametrize("S,H,D,top_k,g,ratio,dtype,seed", CASES[:12])
def test_random_shape_decode_bit_exact(pv, S, H, D, top_k, g, ratio, dtype, seed):
    rng = random.Random(seed)
    B = rng.randint(1, 6)
    gd = rng.choice([1, 2, 3, 4])
    ctx = np.array([rng.choice([1, rng.randint(1, 40), rng.randint(40, 1500)]) for _ in range(B)], np.int64)
    print(f"\n[random decode] B={B} g={gd} ctx={ctx.tolist()} H={H} D={D} k={top_k} r={ratio}", flush=True)
    kc = syn.integers((int(ctx.sum()), H, D), seed + 2, 4, "bf16")
    q = syn.integers((B * gd, H, D), seed + 3, 4, "bf16")
    for mode in ("refine", "reuse"):
        oi, os_ = oracle.decode(q, kc, ctx, gd, top_k, ratio, mode)
        idx, sc = pv.index_decode(dev_tensor(q), dev_tensor(kc), ctx, gd, top_k=top_k, candidate_ratio=ratio,
                                  mode=mode, return_scores=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(parity.to_host(idx), oi)
        np.testing.assert_array_equal(parity.to_host(sc), os_)
