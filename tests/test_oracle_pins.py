"""Pins of the CPU oracle against things other than itself.

Every check here is fixed by the pages or by mathematics, not by re-running
the oracle's own formula:
  * exact rational brute force (tests/exact_ref.py) on tiny integer inputs;
  * closed forms (K, valid counts, proxy rounding);
  * special cases that reduce to a library routine (torch.topk in float64);
  * invariants (causality, uniqueness, padding, order, nesting);
  * a re-expression of the pages' Reuse loop in torch float64;
  * the only value the pages print: the quick test's index shape.
Citations name "PIVOT Explained -- From Paper to Working Code in 10 Minutes"
(sunghee.kr, republished by wpnews.pro) and the arXiv abstract (fugumt.com).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synthetic as syn
from tests import exact_ref

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def valid_counts(row_idx: np.ndarray) -> np.ndarray:
    return (row_idx >= 0).sum(-1)


def check_row_structure(idx, sc, limit_fn):
    """Valid entries first, then -1; distinct; causal (< limit); scores
    non-increasing with ties broken by ascending index; -inf padding."""
    S, H, k = idx.shape
    for i in range(S):
        lim = limit_fn(i)
        for h in range(H):
            r = idx[i, h]
            nv = int((r >= 0).sum())
            assert (r[:nv] >= 0).all() and (r[nv:] == -1).all()
            assert len(set(r[:nv].tolist())) == nv
            assert (r[:nv] < lim).all()
            s = sc[i, h]
            assert np.isneginf(s[nv:]).all()
            for t in range(nv - 1):
                assert s[t] > s[t + 1] or (s[t] == s[t + 1] and r[t] < r[t + 1])


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("top_k,ratio,K", [
    (64, 2.0, 128),     # the code's defaults: K = 2 x top_k ("How It Works")
    (2048, 2.0, 4096),
    (3, 1.5, 4),        # int() truncates 4.5
    (3, 1.1, 3),        # 3.3000000000000003 -> 3
    (10, 2.55, 25),     # 25.499999999999996 -> 25
    (5, 1.0, 5),
    (5, 0.9, -1),       # K < top_k rejected
    (0, 2.0, -1),
])
def test_candidate_count_closed_form(top_k, ratio, K):
    assert oracle.candidate_count(top_k, ratio) == K


def test_quick_test_shape_golden():
    """The quick test of "Show Me The Code" prints the index shape
    (1024, 8, 64); the oracle's output has that shape at those sizes."""
    meta = {}
    with open(os.path.join(GOLDEN, "quick_test_shape.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            for tok in line.split():
                key, val = tok.split("=")
                meta[key] = val
    S, H, D = int(meta["S"]), int(meta["H"]), int(meta["D"])
    shape = tuple(int(x) for x in meta["shape"].split(","))
    cfg = syn.tiny_prefill(integer=False)
    assert cfg["q"].shape == (S, H, D)
    # one head is enough for the shape; the others stay padding
    idx, sc = oracle.prefill(cfg["q"], cfg["k"], int(meta["top_k"]), int(meta["g"]),
                             float(meta["candidate_ratio"]), "refine", heads=(0, 1))
    assert idx.shape == shape
    assert idx.dtype == np.int32


# ---------------------------------------------------- exact brute force

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("S,H,D,top_k,g,ratio", [
    (24, 2, 4, 3, 4, 2.0),
    (19, 1, 8, 4, 4, 1.5),   # ragged last group (m = 3), K = 6
    (16, 2, 4, 2, 1, 2.0),   # g = 1
    (12, 1, 4, 8, 8, 3.0),   # top_k larger than early prefixes
])
def test_oracle_matches_exact_bruteforce(dtype, mode, S, H, D, top_k, g, ratio):
    q = syn.integers((S, H, D), 11 + S, 3, dtype)
    k = syn.integers((S, H, D), 29 + S, 3, dtype)
    K = oracle.candidate_count(top_k, ratio)
    want_idx, want_sc = exact_ref.pivot_exact(q, k, top_k, g, K, mode)
    got_idx, got_sc = oracle.prefill(q, k, top_k, g, ratio, mode)
    np.testing.assert_array_equal(got_idx, want_idx)
    np.testing.assert_array_equal(got_sc.astype(np.float64), want_sc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_matches_exact_bruteforce(dtype):
    q = syn.integers((20, 2, 4), 5, 4, dtype)
    k = syn.integers((20, 2, 4), 6, 4, dtype)
    want_idx, want_sc = exact_ref.dense_exact(q, k, 5)
    got_idx, got_sc = oracle.dense(q, k, 5)
    np.testing.assert_array_equal(got_idx, want_idx)
    np.testing.assert_array_equal(got_sc.astype(np.float64), want_sc)


@pytest.mark.parametrize("m", [3, 5, 6, 7])
def test_proxy_rounding_non_power_of_two_group(m):
    """The proxy of a group of m members is the float32 quotient of the exact
    sum (integer inputs) by m, then RNE to bf16 for bf16 inputs: checked
    bit for bit against a rational-arithmetic rounding."""
    S, H, D = m, 1, 32
    for dtype in ("f32", "bf16"):
        q = syn.integers((S, H, D), 100 + m, 8, dtype)
        got = oracle.proxy(q, m, 0, 0)
        want = exact_ref.proxy_exact(exact_ref.values(q), 0, m, 0, dtype == "bf16")
        np.testing.assert_array_equal(got, np.array([float(w) for w in want], np.float32))


def test_scores_are_rounded_once_from_the_exact_dot():
    """Reported scores equal the exact dot product rounded to float32 (bf16
    inputs: every product is exact in double, so the double sum of 64
    products can differ from the exact value only by double rounding; allow
    one float32 ulp)."""
    S, H, D = 40, 1, 64
    q = syn.gaussian((S, H, D), 3, "bf16")
    k = syn.gaussian((S, H, D), 4, "bf16")
    idx, sc = oracle.dense(q, k, 6)
    qv, kv = exact_ref.values(q), exact_ref.values(k)
    from fractions import Fraction
    for i in range(1, S, 7):
        qi = [Fraction(float(x)) for x in qv[i, 0]]
        for t in range(6):
            c = idx[i, 0, t]
            if c < 0:
                continue
            want = np.float32(exact_ref.dot_f32(qi, kv, c, 0))
            assert abs(int(np.float32(sc[i, 0, t]).view(np.int32)) - int(want.view(np.int32))) <= 1


# ------------------------------------------------------------- invariants

@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_structure_invariants_gaussian(mode):
    S, H, D, top_k, g = 200, 2, 16, 12, 8
    q = syn.gaussian((S, H, D), 21, "bf16")
    k = syn.gaussian((S, H, D), 22, "bf16")
    idx, sc = oracle.prefill(q, k, top_k, g, 2.0, mode)
    check_row_structure(idx, sc, lambda i: max((i // g) * g, 1))
    # valid count = min(top_k, min(K, n_j)) for both modes
    K = 2 * top_k
    for i in range(S):
        n = max((i // g) * g, 1)
        assert (valid_counts(idx[i]) == min(top_k, min(K, n))).all()
    if mode == "reuse":
        for i in range(S):
            j0 = (i // g) * g
            np.testing.assert_array_equal(idx[i], idx[j0])


def test_dense_invariants():
    S, H, D, top_k = 150, 2, 16, 9
    q = syn.gaussian((S, H, D), 31, "f32")
    k = syn.gaussian((S, H, D), 32, "f32")
    idx, sc = oracle.dense(q, k, top_k)
    check_row_structure(idx, sc, lambda i: max(i, 1))
    for i in range(S):
        assert (valid_counts(idx[i]) == min(top_k, max(i, 1))).all()


def test_refine_rows_are_subsets_of_candidates():
    S, H, D, top_k, g = 160, 1, 16, 10, 8
    q = syn.gaussian((S, H, D), 41, "bf16")
    k = syn.gaussian((S, H, D), 42, "bf16")
    idx, _ = oracle.prefill(q, k, top_k, g, 2.0, "refine")
    for j in range(S // g):
        cand, _ = oracle.prefill_candidates(q, k, 0, j, top_k, g, 2.0)
        cs = set(cand.tolist())
        for i in range(j * g, j * g + g):
            r = idx[i, 0]
            assert set(r[r >= 0].tolist()) <= cs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_candidates_match_exact_bruteforce(dtype):
    """C_j (in total order, with proxy scores) of every group equals the
    exact top-K of the exactly rounded proxy over the prefix [0, max(j g, 1)),
    ragged last group included ("How It Works": candidate set of size K)."""
    S, H, D, top_k, g, ratio = 27, 2, 4, 3, 4, 2.0
    q = syn.integers((S, H, D), 71, 3, dtype)
    k = syn.integers((S, H, D), 72, 3, dtype)
    K = oracle.candidate_count(top_k, ratio)
    qv, kv = exact_ref.values(q), exact_ref.values(k)
    for h in range(H):
        for j in range((S + g - 1) // g):
            i0 = j * g
            m = min(g, S - i0)
            p = exact_ref.proxy_exact(qv, i0, m, h, dtype == "bf16")
            want = exact_ref.topk_exact([(exact_ref.dot_f32(p, kv, c, h), c) for c in range(max(i0, 1))], K)
            cand, sc = oracle.prefill_candidates(q, k, h, j, top_k, g, ratio)
            assert cand.tolist() == [c for _, c in want], (h, j)
            assert sc.astype(np.float64).tolist() == [s for s, _ in want], (h, j)


def test_decode_candidates_equal_last_prefill_group():
    """The decode candidate set of sequence b equals that of group L / g of
    a prefill of length L + g whose last g queries are the MTP queries."""
    g, H, D, top_k = 4, 2, 16, 6
    ctx = np.array([40, 8, 64], np.int64)
    B = len(ctx)
    kc = syn.gaussian((int(ctx.sum()), H, D), 131, "bf16")
    qd = syn.gaussian((B * g, H, D), 132, "bf16")
    off = 0
    for b in range(B):
        L = int(ctx[b])
        keys = np.concatenate([kc[off:off + L], syn.gaussian((g, H, D), 133 + b, "bf16")])
        qs = np.concatenate([syn.gaussian((L, H, D), 134 + b, "bf16"), qd[b * g:(b + 1) * g]])
        for h in range(H):
            dc, ds = oracle.decode_candidates(qd, kc, ctx, g, h, b, top_k, 2.0)
            pc, ps = oracle.prefill_candidates(qs, keys, h, L // g, top_k, g, 2.0)
            np.testing.assert_array_equal(dc, pc)
            np.testing.assert_array_equal(ds, ps)
        off += L


# -------------------------------------------------------- special cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_g1_reuse_equals_dense(dtype):
    """With one query per group the proxy is the query itself and the prefix
    is [0, max(i, 1)): Reuse is the dense indexer."""
    S, H, D, top_k = 130, 2, 16, 7
    q = syn.gaussian((S, H, D), 51, dtype)
    k = syn.gaussian((S, H, D), 52, dtype)
    a, sa = oracle.prefill(q, k, top_k, 1, 2.0, "reuse")
    b, sb = oracle.dense(q, k, top_k)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(sa, sb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_g1_refine_equals_dense(dtype):
    S, H, D, top_k = 90, 1, 16, 5
    q = syn.gaussian((S, H, D), 53, dtype)
    k = syn.gaussian((S, H, D), 54, dtype)
    a, _ = oracle.prefill(q, k, top_k, 1, 2.0, "refine")
    b, _ = oracle.dense(q, k, top_k)
    np.testing.assert_array_equal(a, b)


def group_prefix_dense_torch(q, k, top_k, g):
    """Each query ranks the keys [0, max(group_start, 1)) by its own score,
    with torch.topk on float64 values (tie-free inputs)."""
    import torch
    qv = torch.from_numpy(exact_ref.values(q))
    kv = torch.from_numpy(exact_ref.values(k))
    S, H, D = q.shape
    out = np.full((S, H, top_k), -1, np.int64)
    for h in range(H):
        for i in range(S):
            n = max((i // g) * g, 1)
            s = kv[:n, h, :] @ qv[i, h, :]
            kk = min(top_k, n)
            out[i, h, :kk] = torch.topk(s, kk).indices.numpy()
    return out


def test_refine_equals_group_prefix_dense_when_K_covers_prefix():
    """When K >= every prefix length, C is the whole prefix and Refine is each
    query's own top-k over [0, n_j): checked against torch.topk in float64."""
    S, H, D, top_k, g = 96, 2, 16, 6, 8
    q = syn.gaussian((S, H, D), 61, "f32")
    k = syn.gaussian((S, H, D), 62, "f32")
    ratio = float(S)  # K = top_k * S >= S
    idx, _ = oracle.prefill(q, k, top_k, g, ratio, "refine")
    want = group_prefix_dense_torch(q, k, top_k, g)
    np.testing.assert_array_equal(idx, want)


def test_dense_equals_torch_topk_float64():
    import torch
    S, H, D, top_k = 70, 2, 32, 8
    q = syn.gaussian((S, H, D), 71, "f32")
    k = syn.gaussian((S, H, D), 72, "f32")
    idx, _ = oracle.dense(q, k, top_k)
    qv, kv = torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64))
    for h in range(H):
        for i in range(S):
            n = max(i, 1)
            kk = min(top_k, n)
            want = torch.topk(kv[:n, h] @ qv[i, h], kk).indices.numpy()
            np.testing.assert_array_equal(idx[i, h, :kk], want)


def test_refine_with_K_equal_top_k_permutes_reuse():
    S, H, D, top_k, g = 120, 1, 16, 9, 6
    q = syn.gaussian((S, H, D), 81, "bf16")
    k = syn.gaussian((S, H, D), 82, "bf16")
    a, _ = oracle.prefill(q, k, top_k, g, 1.0, "refine")
    b, _ = oracle.prefill(q, k, top_k, g, 1.0, "reuse")
    for i in range(S):
        assert sorted(a[i, 0].tolist()) == sorted(b[i, 0].tolist())


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_zero_queries_tie_break_by_index(mode):
    """Zero queries make every score +-0: the order is by ascending index,
    and -0.0 products (negative keys) must tie with +0.0."""
    S, H, D, top_k, g = 64, 1, 8, 5, 4
    q = np.zeros((S, H, D), np.float32)
    k = syn.integers((S, H, D), 91, 3, "f32")
    idx, sc = oracle.prefill(q, k, top_k, g, 2.0, mode)
    for i in range(S):
        n = max((i // g) * g, 1)
        kk = min(top_k, n)
        np.testing.assert_array_equal(idx[i, 0, :kk], np.arange(kk))
        assert (sc[i, 0, :kk] == 0).all() and not np.signbit(sc[i, 0, :kk]).any()
    didx, _ = oracle.dense(q, k, top_k)
    for i in range(S):
        kk = min(top_k, max(i, 1))
        np.testing.assert_array_equal(didx[i, 0, :kk], np.arange(kk))


def test_first_group_sees_key_zero():
    """Group 0 scans the prefix [0, max(0, 1)) = {0}: its rows are [0, -1, ...]
    (the Reuse code's max(g_start, 1))."""
    q = syn.gaussian((16, 1, 8), 95, "f32")
    k = syn.gaussian((16, 1, 8), 96, "f32")
    for mode in ("refine", "reuse"):
        idx, _ = oracle.prefill(q, k, 4, 4, 2.0, mode)
        for i in range(4):
            np.testing.assert_array_equal(idx[i, 0], [0, -1, -1, -1])


def test_recall_nested_in_K_and_refine_beats_reuse():
    """Top-K sets are nested in K under a total order, so Refine's recall
    against group-prefix dense cannot drop as K grows, and Refine (which
    re-ranks a superset of Reuse's rows) is never below Reuse."""
    S, H, D, top_k, g = 256, 1, 16, 8, 8
    q = syn.ar1_queries(S, H, D, 101, dtype="f32")
    k = syn.pareto_keys(S, H, D, 102, dtype="f32")
    ref = group_prefix_dense_torch(q, k, top_k, g)

    def recall(idx):
        tot = 0.0
        for i in range(g, S):
            a = set(idx[i, 0][idx[i, 0] >= 0].tolist())
            b = set(ref[i, 0][ref[i, 0] >= 0].tolist())
            tot += len(a & b) / len(b)
        return tot / (S - g)

    prev = -1.0
    for ratio in (1.0, 1.5, 2.0, 4.0, 8.0):
        r = recall(oracle.prefill(q, k, top_k, g, ratio, "refine")[0])
        assert r >= prev - 1e-12
        prev = r
    reuse = recall(oracle.prefill(q, k, top_k, g, 2.0, "reuse")[0])
    refine = recall(oracle.prefill(q, k, top_k, g, 2.0, "refine")[0])
    assert refine >= reuse


# ------------------------------------------------- the pages' Reuse loop

def _group_means(qv_h, g):
    """(G, D) means of consecutive blocks of g rows (a shorter last block)."""
    import torch
    S = qv_h.shape[0]
    member_of = torch.arange(S) // g
    G = int(member_of[-1]) + 1
    sums = torch.zeros(G, qv_h.shape[1], dtype=torch.float64).index_add_(0, member_of, qv_h)
    return sums / torch.bincount(member_of, minlength=G)[:, None].double(), member_of


def _ranked(scores):
    """Column order of each row by descending score, earlier column first on
    equal scores (a stable sort)."""
    import torch
    return torch.argsort(scores, dim=1, descending=True, stable=True)


def pages_reuse_torch(q, k, top_k, group_size, candidate_ratio):
    """PIVOT-Reuse by its definition ("Show Me The Code", pivot_reuse),
    vectorised per head in torch float64: all group means at once, one
    prefix-masked score matrix (group j sees keys [0, max(j*g, 1))), every
    row ranked, and each member takes its group's first min(top_k, K, n_j)
    keys. Unfilled slots hold 0, as the pages' zero-initialised output does."""
    import torch
    qv = torch.from_numpy(exact_ref.values(q))
    kv = torch.from_numpy(exact_ref.values(k))
    S, H, D = q.shape
    n_cand = int(top_k * candidate_ratio)
    res = torch.zeros(S, H, top_k, dtype=torch.long)
    slot = torch.arange(top_k)
    for head in range(H):
        means, member_of = _group_means(qv[:, head], group_size)
        seen = torch.clamp(torch.arange(means.shape[0]) * group_size, min=1)
        sc = means @ kv[:, head].T
        sc[torch.arange(S)[None, :] >= seen[:, None]] = -torch.inf
        lead = _ranked(sc)[:, :top_k]
        take = torch.minimum(torch.minimum(seen, torch.tensor(n_cand)), torch.tensor(top_k))
        lead = torch.where(slot[None, :] < take[:, None], lead, 0)
        res[:, head] = lead[member_of]
    return res.numpy()


def test_reuse_matches_pages_loop_float64():
    """On tie-free fp32 inputs with power-of-two groups the proxy is exact
    in float32 up to the one division, and the pages' float64 loop and the
    oracle agree on every row once -1 padding is mapped to the pages' 0."""
    S, H, D, top_k, g = 128, 2, 16, 6, 8
    q = syn.integers((S, H, D), 111, 8, "f32")  # exact float32 means (g = 8)
    k = syn.gaussian((S, H, D), 112, "f32")
    idx, _ = oracle.prefill(q, k, top_k, g, 2.0, "reuse")
    want = pages_reuse_torch(q, k, top_k, g, 2.0)
    np.testing.assert_array_equal(np.where(idx < 0, 0, idx), want)


# ------------------------------- literal per-position Refine (comparison)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,H,D,top_k,g,ratio", [
    (24, 2, 4, 3, 4, 2.0),
    (19, 1, 8, 4, 4, 1.5),   # ragged last group
    (12, 1, 4, 8, 8, 3.0),   # top_k larger than early prefixes
])
def test_literal_refine_matches_exact_bruteforce(dtype, S, H, D, top_k, g, ratio):
    q = syn.integers((S, H, D), 41 + S, 3, dtype)
    k = syn.integers((S, H, D), 43 + S, 3, dtype)
    K = oracle.candidate_count(top_k, ratio)
    want_idx, want_sc = exact_ref.literal_exact(q, k, top_k, g, K)
    got_idx, got_sc = oracle.prefill(q, k, top_k, g, ratio, "refine_literal")
    np.testing.assert_array_equal(got_idx, want_idx)
    np.testing.assert_array_equal(got_sc.astype(np.float64), want_sc)


def test_literal_refine_identities():
    """Position i of the literal loop scans [0, i): at a group's first
    member (i = j*g, j >= 1) that is the one-scan prefix, so the rows agree;
    with g = 1 the proxy is q_i itself and every row i >= 1 is the dense row;
    row 0 is padding."""
    S, H, D, top_k, g = 96, 2, 16, 5, 8
    q = syn.gaussian((S, H, D), 51, "f32")
    k = syn.gaussian((S, H, D), 52, "f32")
    lit, lsc = oracle.prefill(q, k, top_k, g, 2.0, "refine_literal")
    one, osc = oracle.prefill(q, k, top_k, g, 2.0, "refine")
    firsts = np.arange(g, S, g)
    np.testing.assert_array_equal(lit[firsts], one[firsts])
    np.testing.assert_array_equal(lsc[firsts], osc[firsts])
    assert (lit[0] == -1).all() and np.isneginf(lsc[0]).all()
    lit1, _ = oracle.prefill(q, k, top_k, 1, 2.0, "refine_literal")
    dense, _ = oracle.dense(q, k, top_k)
    np.testing.assert_array_equal(lit1[1:], dense[1:])
    # K covering every prefix: the candidate set is the whole prefix
    litK, _ = oracle.prefill(q, k, 2, g, float(S), "refine_literal")
    denseK, _ = oracle.dense(q, k, 2)
    np.testing.assert_array_equal(litK[1:], denseK[1:])


def pages_refine_torch(q, k, top_k, group_size, candidate_ratio):
    """The per-position Refine of "Show Me The Code" (pivot_refine as
    written), by its definition and vectorised per head in torch float64:
    position p ranks keys [0, p) by its group's mean, keeps the first
    min(K, p) as its candidates, ranks those by q_p and keeps the first
    min(top_k, |C|). Position 0 has no key before it and stays zero, like
    every unfilled slot of the pages' zero-initialised output."""
    import torch
    qv = torch.from_numpy(exact_ref.values(q))
    kv = torch.from_numpy(exact_ref.values(k))
    S, H, D = q.shape
    n_cand = int(top_k * candidate_ratio)
    res = torch.zeros(S, H, top_k, dtype=torch.long)
    pos = torch.arange(S)
    for head in range(H):
        means, member_of = _group_means(qv[:, head], group_size)
        sc = means[member_of] @ kv[:, head].T                  # (S, S) by each position's group mean
        sc[pos[None, :] >= pos[:, None]] = -torch.inf          # keys strictly before the position
        cand = _ranked(sc)[:, :n_cand]                         # (S, K)
        n_c = torch.minimum(pos, torch.tensor(n_cand))
        ok = torch.arange(cand.shape[1])[None, :] < n_c[:, None]
        own = torch.einsum("pcd,pd->pc", kv[:, head][cand], qv[:, head])
        own = torch.where(ok, own, -torch.inf)
        pick = torch.gather(cand, 1, _ranked(own)[:, :top_k])
        keep = torch.minimum(n_c, torch.tensor(top_k))
        pick = torch.where(torch.arange(pick.shape[1])[None, :] < keep[:, None], pick, 0)
        res[:, head, :pick.shape[1]] = pick
    return res.numpy()


def test_literal_refine_matches_pages_loop_float64():
    """Tie-free fp32 inputs, power-of-two groups: the pages' float64 loop and
    the oracle's literal mode agree on every row once -1 padding is mapped
    to the pages' 0."""
    S, H, D, top_k, g = 96, 2, 16, 6, 8
    q = syn.integers((S, H, D), 121, 8, "f32")
    k = syn.gaussian((S, H, D), 122, "f32")
    idx, _ = oracle.prefill(q, k, top_k, g, 2.0, "refine_literal")
    want = pages_refine_torch(q, k, top_k, g, 2.0)
    np.testing.assert_array_equal(np.where(idx < 0, 0, idx), want)


def test_literal_rows_api_matches_full():
    S, H, D, top_k, g = 64, 3, 8, 4, 4
    q = syn.gaussian((S, H, D), 61, "bf16")
    k = syn.gaussian((S, H, D), 62, "bf16")
    full, fsc = oracle.prefill(q, k, top_k, g, 2.0, "refine_literal")
    ri = np.array([0, 1, 5, 17, 63], np.int64)
    rh = np.array([0, 2, 1, 0, 2], np.int32)
    idx, sc = oracle.prefill_rows(q, k, ri, rh, top_k, g, 2.0, "refine_literal")
    np.testing.assert_array_equal(idx, full[ri, rh])
    np.testing.assert_array_equal(sc, fsc[ri, rh])


# ----------------------------------------------------------- decode path

@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_decode_equals_last_prefill_group(mode):
    """A decode step of g queries after a context of length L (L % g == 0) is
    the group j = L / g of a prefill of length L + g whose last g queries are
    the MTP queries (the abstract: one algorithm, groups formed differently)."""
    g, H, D, top_k = 4, 2, 16, 6
    ctx = np.array([40, 8, 64], np.int64)
    B = len(ctx)
    kc = syn.gaussian((int(ctx.sum()), H, D), 121, "bf16")
    qd = syn.gaussian((B * g, H, D), 122, "bf16")
    idx, sc = oracle.decode(qd, kc, ctx, g, top_k, 2.0, mode)
    off = 0
    for b in range(B):
        L = int(ctx[b])
        keys = np.concatenate([kc[off:off + L], syn.gaussian((g, H, D), 123 + b, "bf16")])
        qs = np.concatenate([syn.gaussian((L, H, D), 124 + b, "bf16"), qd[b * g:(b + 1) * g]])
        pidx, psc = oracle.prefill(qs, keys, top_k, g, 2.0, mode)
        np.testing.assert_array_equal(idx[b * g:(b + 1) * g], pidx[L:L + g])
        np.testing.assert_array_equal(sc[b * g:(b + 1) * g], psc[L:L + g])
        off += L


def test_rows_api_matches_full():
    S, H, D, top_k, g = 100, 3, 16, 7, 8
    q = syn.gaussian((S, H, D), 131, "bf16")
    k = syn.gaussian((S, H, D), 132, "bf16")
    rng = np.random.default_rng(0)
    ri = rng.integers(0, S, 40)
    rh = rng.integers(0, H, 40)
    for mode in ("refine", "reuse"):
        full, fs = oracle.prefill(q, k, top_k, g, 2.0, mode)
        rows, rs = oracle.prefill_rows(q, k, ri, rh, top_k, g, 2.0, mode)
        np.testing.assert_array_equal(rows, full[ri, rh])
        np.testing.assert_array_equal(rs, fs[ri, rh])
    fd, _ = oracle.dense(q, k, top_k)
    rd, _ = oracle.dense_rows(q, k, ri, rh, top_k)
    np.testing.assert_array_equal(rd, fd[ri, rh])


def test_groups_api_matches_full():
    S, H, D, top_k, g = 90, 2, 16, 6, 8   # ragged last group
    q = syn.gaussian((S, H, D), 141, "bf16")
    k = syn.gaussian((S, H, D), 142, "bf16")
    heads = np.array([0, 1, 1, 0], np.int32)
    groups = np.array([0, 5, 11, 7], np.int64)
    for mode in ("refine", "reuse"):
        full, fs = oracle.prefill(q, k, top_k, g, 2.0, mode)
        gi, gs = oracle.prefill_groups(q, k, heads, groups, top_k, g, 2.0, mode)
        for t in range(len(heads)):
            i0 = groups[t] * g
            m = min(g, S - i0)
            np.testing.assert_array_equal(gi[t, :m], full[i0:i0 + m, heads[t]])
            np.testing.assert_array_equal(gs[t, :m], fs[i0:i0 + m, heads[t]])
            assert (gi[t, m:] == -1).all()


# ------------------------------------------- downstream sparse attention

def _att_inputs(S=40, H=2, D=8, seed=71, dtype="f32"):
    q = syn.gaussian((S, H, D), seed, dtype)
    k = syn.gaussian((S, H, D), seed + 1, dtype)
    v = syn.gaussian((S, H, D), seed + 2, dtype)
    return q, k, v


def test_attention_zero_query_is_the_mean_of_v():
    """q = 0: every weight is equal, the output is the mean of V[idx]."""
    q, k, v = _att_inputs()
    q[:] = 0
    rng = np.random.default_rng(3)
    idx = np.stack([np.stack([rng.choice(40, 5, replace=False) for _ in range(2)]) for _ in range(40)]).astype(np.int32)
    out = oracle.sparse_attention(q, k, v, idx)
    want = np.stack([[v[idx[i, h], h].astype(np.float64).mean(axis=0) for h in range(2)] for i in range(40)])
    np.testing.assert_allclose(out, want, rtol=1e-6, atol=1e-7)


def test_attention_single_index_returns_that_value_row():
    q, k, v = _att_inputs(dtype="bf16")
    idx = np.full((40, 2, 4), -1, np.int32)
    idx[:, :, 2] = (np.arange(40) * 7 % 40)[:, None]
    out = oracle.sparse_attention(q, k, v, idx)
    vv = exact_ref.values(v)
    want = np.stack([[vv[(i * 7) % 40, h] for h in range(2)] for i in range(40)])
    np.testing.assert_array_equal(out, want.astype(np.float32))


def test_attention_padding_order_and_empty_rows():
    """-1 and out-of-range entries are padding; the order of the entries does
    not matter (up to rounding); a row without entries is zero."""
    q, k, v = _att_inputs()
    rng = np.random.default_rng(5)
    base = np.stack([np.stack([rng.choice(40, 6, replace=False) for _ in range(2)]) for _ in range(40)]).astype(np.int32)
    a = oracle.sparse_attention(q, k, v, base)
    padded = np.concatenate([base[:, :, :3], np.full((40, 2, 2), -1, np.int32), base[:, :, 3:],
                             np.full((40, 2, 1), 40, np.int32)], axis=2)
    np.testing.assert_array_equal(oracle.sparse_attention(q, k, v, padded), a)
    perm = base[:, :, ::-1].copy()
    np.testing.assert_allclose(oracle.sparse_attention(q, k, v, perm), a, rtol=1e-6, atol=1e-7)
    empty = np.full((40, 2, 3), -1, np.int32)
    assert (oracle.sparse_attention(q, k, v, empty) == 0).all()


def test_attention_two_keys_is_a_logistic_weight():
    """Two entries: w_1 = 1 / (1 + exp(-scale (s_1 - s_2)))."""
    q, k, v = _att_inputs(S=16, H=1, D=4)
    idx = np.zeros((16, 1, 2), np.int32)
    idx[:, 0, 0] = 3
    idx[:, 0, 1] = 11
    out = oracle.sparse_attention(q, k, v, idx)
    qv, kv, vv = (a.astype(np.float64) for a in (q, k, v))
    for i in range(16):
        d = (qv[i, 0] @ kv[3, 0] - qv[i, 0] @ kv[11, 0]) * 0.5
        w = 1.0 / (1.0 + np.exp(-d))
        np.testing.assert_allclose(out[i, 0], w * vv[3, 0] + (1 - w) * vv[11, 0], rtol=1e-6, atol=1e-7)


def test_attention_large_scale_selects_the_argmax():
    q, k, v = _att_inputs(S=32, H=1, D=8)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(32, 8, replace=False) for _ in range(32)])[:, None, :].astype(np.int32)
    out = oracle.sparse_attention(q, k, v, idx, scale=1e6)
    qv, kv = q.astype(np.float64), k.astype(np.float64)
    for i in range(32):
        s = kv[idx[i, 0], 0] @ qv[i, 0]
        np.testing.assert_array_equal(out[i, 0], v[idx[i, 0, np.argmax(s)], 0])


def test_attention_matches_pages_demo_loop_float64():
    """The pages' quick-test attention loop in torch float64 (positions >= 1;
    full index rows, no padding)."""
    import torch
    import torch.nn.functional as F
    S, H, D, top_k = 64, 2, 16, 6
    q, k, v = _att_inputs(S, H, D, 81)
    rng = np.random.default_rng(4)
    idx = np.stack([np.stack([rng.choice(S, top_k, replace=False) for _ in range(H)]) for _ in range(S)]).astype(np.int32)
    out = oracle.sparse_attention(q, k, v, idx)
    qt, kt, vt = (torch.from_numpy(a.astype(np.float64)) for a in (q, k, v))
    it = torch.from_numpy(idx.astype(np.int64))
    scale = D ** -0.5
    for pos in range(1, S):
        for h in range(H):
            sel = it[pos, h]
            w = F.softmax(qt[pos, h] @ kt[sel, h].T * scale, dim=-1)
            np.testing.assert_allclose(out[pos, h], (w @ vt[sel, h]).numpy(), rtol=1e-6, atol=1e-7)


def test_attention_rows_api_matches_full():
    q, k, v = _att_inputs(S=48, H=3, D=8, seed=91, dtype="bf16")
    rng = np.random.default_rng(12)
    idx = rng.integers(-1, 48, (48, 3, 7)).astype(np.int32)
    full = oracle.sparse_attention(q, k, v, idx)
    ri = np.array([0, 5, 47, 20], np.int64)
    rh = np.array([2, 0, 1, 2], np.int32)
    rows = oracle.sparse_attention_rows(q, k, v, idx[ri, rh], ri, rh)
    np.testing.assert_array_equal(rows, full[ri, rh])
