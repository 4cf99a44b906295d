"""GPU parity of the downstream sparse attention (the pages' quick-test
attention over indexer rows) against the oracle.

Tolerance, from the arithmetic: the GPU forms each score as a float32 dot of
D products and applies the softmax in float32 (base-2 exponentials); the dot
can be off by about D * 2^-24 * |q| |k|, which moves every weight by that
much times `scale` in relative terms. A row's output may therefore differ by
  max|v| * (1e-4 + 8 * D * 2^-24 * scale * max_c |q| |k_c|)
(max over the row's valid entries).
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


def dev_tensor(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def row_bounds(qv, kv, vv, idx, rows_i, rows_h, scale):
    S, H, D = qv.shape
    out = np.empty(len(rows_i))
    for r, (i, h) in enumerate(zip(rows_i, rows_h)):
        c = idx[r]
        c = c[(c >= 0) & (c < S)]
        if len(c) == 0:
            out[r] = 1e-30
            continue
        qk = np.linalg.norm(qv[i, h]) * np.linalg.norm(kv[c, h], axis=1).max()
        out[r] = np.abs(vv[c, h]).max() * (1e-4 + 8 * D * 2.0 ** -24 * scale * qk)
    return out


def check_rows(got, want, bounds):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64)).max(axis=1)
    bad = np.nonzero(err > bounds)[0]
    assert len(bad) == 0, [(int(b), float(err[b]), float(bounds[b])) for b in bad[:5]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_on_indexer_rows_matches_oracle(pv, dtype, D):
    """Indices from the Refine indexer (top_k = 40, not a multiple of 16),
    with planted padding, out-of-range entries and repeats."""
    print(f"\n[attention] D={D} {dtype}", flush=True)
    S, H, top_k = 700, 3, 40
    q = syn.gaussian((S, H, D), 301 + D, dtype)
    k = syn.gaussian((S, H, D), 302 + D, dtype)
    v = syn.gaussian((S, H, D), 303 + D, dtype)
    qd, kd, vd = dev_tensor(q), dev_tensor(k), dev_tensor(v)
    idx = pv.index_prefill(qd, kd, top_k=top_k, g=8, mode="refine")
    torch.cuda.synchronize()
    ih = parity.to_host(idx).copy()
    rng = np.random.default_rng(D)
    ih[rng.integers(0, S, 50), rng.integers(0, H, 50), rng.integers(0, top_k, 50)] = S + 3   # out of range
    ih[rng.integers(0, S, 50), rng.integers(0, H, 50), 7] = ih[0, 0, 0]                     # repeats / any key
    ih[5, 1, :] = -1                                                                          # empty row
    idx_d = torch.from_numpy(ih).to(DEV)
    out = pv.sparse_attention(qd, kd, vd, idx_d)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.sparse_attention(q, k, v, ih)
    assert (got[5, 1] == 0).all()
    ri = np.repeat(np.arange(S), H)
    rh = np.tile(np.arange(H), S).astype(np.int32)
    qv, kv, vv = (syn.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a for a in (q, k, v))
    bounds = row_bounds(qv, kv, vv, ih.reshape(S * H, top_k), ri, rh, D ** -0.5)
    check_rows(got.reshape(S * H, D), want.reshape(S * H, D), bounds)


def test_attention_full_size_sampled_rows(pv):
    """The 64K workload's distribution (AR(1) queries, Pareto-norm keys and
    values) on 8 heads with the Refine indexer's rows (top_k = 2048);
    sampled rows against the oracle."""
    S, H, g, top_k = 65536, 8, 8, 2048
    print(f"\n[attention] S={S} H={H} top_k={top_k}", flush=True)
    cfg = syn.long_prefill_device(DEV, S=S, H=H, g=g, seed=1008)
    q, k = cfg["q"], cfg["k"]
    v = syn.pareto_keys_device(S, H, 128, 2008, DEV)
    idx = pv.index_prefill(q, k, top_k=top_k, g=g, mode="refine")
    out = pv.sparse_attention(q, k, v, idx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    ri = np.concatenate([rng.integers(0, S, 40), [0, 1, S - 1]])
    rh = rng.integers(0, H, len(ri)).astype(np.int32)
    ri_d = torch.from_numpy(ri).to(DEV)
    rh_d = torch.from_numpy(rh.astype(np.int64)).to(DEV)
    got = out[ri_d, rh_d].cpu().numpy()
    irows = idx[ri_d, rh_d].cpu().numpy()
    del out, idx
    qh, kh, vh = (syn.bf16_tensor_to_bits(t) for t in (q, k, v))
    want = oracle.sparse_attention_rows(qh, kh, vh, irows, ri, rh)
    qv, kv, vv = (syn.bf16_bits_to_f32(a) for a in (qh, kh, vh))
    check_rows(got, want, row_bounds(qv, kv, vv, irows, ri, rh, 128 ** -0.5))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("g", [8, 3, 16])
def test_grouped_attention_on_reuse_rows_matches_oracle(pv, dtype, D, g):
    """Rows shared by groups of g positions (Reuse rows; g = 16 takes two
    blocks per group, g = 3 leaves a ragged last group), top_k = 100 (not a
    multiple of the 64-entry chunk), with planted padding, out-of-range
    entries, repeats and an empty group row. Expected: the oracle's
    attention with every member given its group's first row."""
    print(f"\n[grouped attention] D={D} {dtype} g={g}", flush=True)
    S, H, top_k = 700, 3, 100
    q = syn.gaussian((S, H, D), 401 + D + g, dtype)
    k = syn.gaussian((S, H, D), 402 + D + g, dtype)
    v = syn.gaussian((S, H, D), 403 + D + g, dtype)
    qd, kd, vd = dev_tensor(q), dev_tensor(k), dev_tensor(v)
    idx = pv.index_prefill(qd, kd, top_k=top_k, g=g, mode="reuse")
    torch.cuda.synchronize()
    ih = parity.to_host(idx).copy()
    rng = np.random.default_rng(D + g)
    firsts = np.arange(0, S, g)
    ih[rng.choice(firsts, 30), rng.integers(0, H, 30), rng.integers(0, top_k, 30)] = S + 5    # out of range
    ih[rng.choice(firsts, 30), rng.integers(0, H, 30), 9] = ih[g, 0, 0]                      # repeats
    ih[firsts[7], 2, :] = -1                                                                  # empty group row
    idx_d = torch.from_numpy(ih).to(DEV)
    out = pv.sparse_attention(qd, kd, vd, idx_d, g=g)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    shared = ih[(np.arange(S) // g) * g]          # each member's row: its group's first
    want = oracle.sparse_attention(q, k, v, shared)
    e0 = firsts[7]
    assert (got[e0:e0 + g, 2] == 0).all()
    ri = np.repeat(np.arange(S), H)
    rh = np.tile(np.arange(H), S).astype(np.int32)
    qv, kv, vv = (syn.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a for a in (q, k, v))
    bounds = row_bounds(qv, kv, vv, shared.reshape(S * H, top_k), ri, rh, D ** -0.5)
    check_rows(got.reshape(S * H, D), want.reshape(S * H, D), bounds)


def test_grouped_attention_full_size_reuse_rows(pv):
    """Reuse rows (top_k = 2048, g = 8) of the 64K workload's distribution on
    8 heads: sampled rows of the grouped attention against the oracle."""
    S, H, g, top_k = 65536, 8, 8, 2048
    print(f"\n[grouped attention] S={S} H={H} top_k={top_k}", flush=True)
    cfg = syn.long_prefill_device(DEV, S=S, H=H, g=g, seed=1009)
    q, k = cfg["q"], cfg["k"]
    v = syn.pareto_keys_device(S, H, 128, 2009, DEV)
    idx = pv.index_prefill(q, k, top_k=top_k, g=g, mode="reuse")
    out = pv.sparse_attention(q, k, v, idx, g=g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(23)
    ri = np.concatenate([rng.integers(0, S, 40), [0, 1, 7, 8, S - 1]])
    rh = rng.integers(0, H, len(ri)).astype(np.int32)
    ri_d = torch.from_numpy(ri).to(DEV)
    rh_d = torch.from_numpy(rh.astype(np.int64)).to(DEV)
    got = out[ri_d, rh_d].cpu().numpy()
    first_d = torch.from_numpy((ri // g) * g).to(DEV)
    irows = idx[first_d, rh_d].cpu().numpy()
    del out, idx
    qh, kh, vh = (syn.bf16_tensor_to_bits(t) for t in (q, k, v))
    want = oracle.sparse_attention_rows(qh, kh, vh, irows, ri, rh)
    qv, kv, vv = (syn.bf16_bits_to_f32(a) for a in (qh, kh, vh))
    check_rows(got, want, row_bounds(qv, kv, vv, irows, ri, rh, 128 ** -0.5))
