"""GPU parity at the full workload sizes, on sampled rows the oracle
computes one by one (in the same launch configuration the bench times).

  * S=16384, H=16, D=128 bf16 integers in [-4, 4], top_k=512, g=8, K=1024:
    every float32 score is exact, so sampled rows are compared bit for bit;
    every row's structure (padding, causality, uniqueness) is checked.
  * S=65536, H=64 and S=131072, H=32 (D=128 bf16, AR(1) queries,
    Pareto-norm keys, top_k=2048, K=4096): sampled rows, tie-tolerant.
  * decode: 64 sequences with contexts U[32768, 131072], H=8, g in {2, 4}:
    every sequence of one head against the oracle, tie-tolerant.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def pv():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import top_token_selection_amd as pv
    return pv


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_int_workload_sampled_rows_bit_exact(pv, mode):
    print(f"\n[int workload] S=16384 H=16 {mode}", flush=True)
    cfg = syn.int_prefill()
    q, k, top_k, g = cfg["q"], cfg["k"], cfg["top_k"], cfg["g"]
    S, H, D = q.shape
    idx, sc = pv.index_prefill(to_dev(q), to_dev(k), top_k=top_k, g=g, mode=mode, return_scores=True)
    torch.cuda.synchronize()
    gi, gs = parity.to_host(idx), parity.to_host(sc)
    K = 2 * top_k
    lim = np.maximum((np.arange(S) // g) * g, 1)[:, None]
    parity.structure_ok(gi, gs, lim, np.minimum(top_k, np.minimum(K, lim)))
    rng = np.random.default_rng(3)
    ri = np.concatenate([rng.integers(0, S, 120), [0, 1, 7, 8, 9, 1023, 1024, 1025, S - 1]])
    rh = rng.integers(0, H, len(ri)).astype(np.int32)
    oi, os_ = oracle.prefill_rows(q, k, ri, rh, top_k, g, 2.0, mode)
    np.testing.assert_array_equal(gi[ri, rh], oi)
    np.testing.assert_array_equal(gs[ri, rh], os_)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_int_workload_index_only_bit_exact(pv, mode):
    """Index-only rows (wavefront bucket sorts) on the integer workload."""
    print(f"\n[int workload] S=16384 H=16 {mode} index-only", flush=True)
    cfg = syn.int_prefill()
    q, k, top_k, g = cfg["q"], cfg["k"], cfg["top_k"], cfg["g"]
    S, H, D = q.shape
    idx = pv.index_prefill(to_dev(q), to_dev(k), top_k=top_k, g=g, mode=mode)
    torch.cuda.synchronize()
    gi = parity.to_host(idx)
    rng = np.random.default_rng(4)
    ri = np.concatenate([rng.integers(0, S, 120), [0, 1, 7, 8, 9, 1023, 1024, 1025, S - 1]])
    rh = rng.integers(0, H, len(ri)).astype(np.int32)
    oi, _ = oracle.prefill_rows(q, k, ri, rh, top_k, g, 2.0, mode)
    np.testing.assert_array_equal(gi[ri, rh], oi)


@pytest.mark.parametrize("long", [False, True])
@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_long_workload_index_only_equals_scored(pv, mode, long):
    """At full size, the index-only launch (the bench's: wavefront bucket
    sorts) returns exactly the indices of the launch that also returns scores
    (general selectors), in every row."""
    S, H, g, seed = (131072, 32, 16, 1004) if long else (65536, 64, 8, 1003)
    print(f"\n[long workload] S={S} H={H} g={g} {mode} index-only vs scored", flush=True)
    cfg = syn.long_prefill_device(DEV, S=S, H=H, g=g, seed=seed)
    q, k, top_k = cfg["q"], cfg["k"], cfg["top_k"]
    a = pv.index_prefill(q, k, top_k=top_k, g=g, mode=mode)
    b, sc = pv.index_prefill(q, k, top_k=top_k, g=g, mode=mode, return_scores=True)
    del sc
    torch.cuda.synchronize()
    same = torch.eq(a, b).all(dim=2)
    bad = torch.nonzero(~same)[:5].tolist()
    assert not bad, bad


@pytest.mark.parametrize("long", [False, True])
@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_long_workloads_sampled_rows_tolerant(pv, mode, long):
    S, H, g, seed = (131072, 32, 16, 1004) if long else (65536, 64, 8, 1003)
    print(f"\n[long workload] S={S} H={H} g={g} {mode}", flush=True)
    cfg = syn.long_prefill_device(DEV, S=S, H=H, g=g, seed=seed)
    q, k, top_k = cfg["q"], cfg["k"], cfg["top_k"]
    D = q.shape[2]
    idx, sc = pv.index_prefill(q, k, top_k=top_k, g=g, mode=mode, return_scores=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    n_rows = 24
    ri = np.concatenate([rng.integers(0, S, n_rows - 4), [1, g * 600, S // 2, S - 1]])
    rh = rng.integers(0, H, n_rows).astype(np.int32)
    ri_d = torch.from_numpy(ri).to(DEV)
    rh_d = torch.from_numpy(rh.astype(np.int64)).to(DEV)
    gi = idx[ri_d, rh_d].cpu().numpy()
    gs = sc[ri_d, rh_d].cpu().numpy()
    del idx, sc
    qh = syn.bf16_tensor_to_bits(q)
    kh = syn.bf16_tensor_to_bits(k)
    oi, os_ = oracle.prefill_rows(qh, kh, ri, rh, top_k, g, 2.0, mode)
    errs = []
    for r in range(n_rows):
        i, h = int(ri[r]), int(rh[r])
        j = i // g
        proxy = oracle.proxy(qh, g, h, j).astype(np.float64)
        cand = csc = None
        if mode == "refine":
            cand, csc = oracle.prefill_candidates(qh, kh, h, j, top_k, g, 2.0)
            avec = syn.bf16_bits_to_f32(qh[i, h]).astype(np.float64)
        else:
            avec = proxy
        e = parity.tolerant_row_match(gi[r], gs[r], oi[r], os_[r], avec, kh, h, D,
                                      cand_idx=cand, cand_sc=csc, proxy=proxy)
        if e:
            errs.append((i, h, e))
    assert not errs, errs[:5]


def test_dense_index_only_equals_scored(pv):
    """The dense indexer at S=32768, H=4 on the long-workload distribution:
    index-only rows (one wavefront per query row) equal the scored launch's
    (block selector) in every row."""
    print("\n[dense] S=32768 H=4 index-only vs scored", flush=True)
    cfg = syn.long_prefill_device(DEV, S=32768, H=4, g=8, seed=1006)
    q, k, top_k = cfg["q"], cfg["k"], cfg["top_k"]
    a = pv.dense_index(q, k, top_k=top_k)
    b, sc = pv.dense_index(q, k, top_k=top_k, return_scores=True)
    del sc
    torch.cuda.synchronize()
    bad = torch.nonzero(~torch.eq(a, b).all(dim=2))[:5].tolist()
    assert not bad, bad


@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_decode_workload_tolerant(pv, mode, g):
    print(f"\n[decode workload] g={g} {mode}", flush=True)
    dc = syn.decode_step_device(DEV, g=g)
    q, kc, ctx, top_k = dc["q"], dc["k_cache"], dc["ctx_lens"], dc["top_k"]
    idx, sc = pv.index_decode(q, kc, ctx, g, top_k=top_k, mode=mode, return_scores=True)
    torch.cuda.synchronize()
    h = 3
    gi = idx[:, h].cpu().numpy()
    gs = sc[:, h].cpu().numpy()
    qh = syn.bf16_tensor_to_bits(q[:, h:h + 1].contiguous())
    kh = syn.bf16_tensor_to_bits(kc[:, h:h + 1].contiguous())
    del idx, sc
    oi, os_ = oracle.decode(qh, kh, ctx, g, top_k, 2.0, mode)
    D = q.shape[2]
    errs = []
    off = 0
    for b in range(len(ctx)):
        n = int(ctx[b])
        qv = syn.bf16_bits_to_f32(qh[b * g:(b + 1) * g, 0]).astype(np.float64)
        # proxy: float32 sum, one float32 division, bf16 rounding
        ps = np.zeros(D, np.float32)
        for t in range(g):
            ps = (ps + qv[t].astype(np.float32)).astype(np.float32)
        proxy = syn.bf16_bits_to_f32(syn.to_bf16_bits(ps / np.float32(g))).astype(np.float64)
        kslice = kh[off:off + n]
        cand = csc = None
        if mode == "refine":
            kv = syn.bf16_bits_to_f32(kslice[:, 0]).astype(np.float64)
            ps_all = kv @ proxy
            order = np.lexsort((np.arange(n), -ps_all))
            cand = order[:min(2 * top_k, n)]
            csc = ps_all[cand]
        for t in range(g):
            r = b * g + t
            avec = qv[t] if mode == "refine" else proxy
            e = parity.tolerant_row_match(gi[r], gs[r], oi[r, 0], os_[r, 0], avec, kslice, 0, D,
                                          cand_idx=cand, cand_sc=csc, proxy=proxy)
            if e:
                errs.append((b, t, e))
        off += n
    assert not errs, errs[:5]


def test_literal_refine_long_distribution_tolerant(pv):
    """The per-position rescan at S=16384, H=8 on the long-workload
    distribution (AR(1) queries, Pareto-norm keys, top_k=2048, K=4096):
    sampled rows against the oracle, tie-tolerant; the index-only launch
    equals the scored one in every row."""
    S, H, g = 16384, 8, 8
    print(f"\n[literal] S={S} H={H} g={g}", flush=True)
    cfg = syn.long_prefill_device(DEV, S=S, H=H, g=g, seed=1007)
    q, k, top_k = cfg["q"], cfg["k"], cfg["top_k"]
    D = q.shape[2]
    idx, sc = pv.index_prefill(q, k, top_k=top_k, g=g, mode="refine_literal", return_scores=True)
    only = pv.index_prefill(q, k, top_k=top_k, g=g, mode="refine_literal")
    torch.cuda.synchronize()
    bad = torch.nonzero(~torch.eq(idx, only).all(dim=2))[:5].tolist()
    assert not bad, bad
    rng = np.random.default_rng(8)
    ri = np.concatenate([rng.integers(0, S, 12), [0, 1, 9, 4097, S - 1]])
    rh = rng.integers(0, H, len(ri)).astype(np.int32)
    ri_d = torch.from_numpy(ri).to(DEV)
    rh_d = torch.from_numpy(rh.astype(np.int64)).to(DEV)
    gi = idx[ri_d, rh_d].cpu().numpy()
    gs = sc[ri_d, rh_d].cpu().numpy()
    del idx, sc, only
    qh = syn.bf16_tensor_to_bits(q)
    kh = syn.bf16_tensor_to_bits(k)
    oi, os_ = oracle.prefill_rows(qh, kh, ri, rh, top_k, g, 2.0, "refine_literal")
    errs = []
    for r in range(len(ri)):
        i, h = int(ri[r]), int(rh[r])
        if i == 0:
            assert (gi[r] == -1).all(), gi[r][:4]
            continue
        j = i // g
        proxy = oracle.proxy(qh, g, h, j).astype(np.float64)
        kv = syn.bf16_bits_to_f32(kh[:i, h]).astype(np.float64)
        ps = kv @ proxy
        order = np.lexsort((np.arange(i), -ps))
        cand = order[:min(4096, i)]
        avec = syn.bf16_bits_to_f32(qh[i, h]).astype(np.float64)
        e = parity.tolerant_row_match(gi[r], gs[r], oi[r], os_[r], avec, kh, h, D,
                                      cand_idx=cand, cand_sc=ps[cand], proxy=proxy)
        if e:
            errs.append((i, h, e))
    assert not errs, errs[:5]
