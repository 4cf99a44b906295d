"""The tie-tolerant comparator (tests/parity.py) on the CPU: it accepts the
oracle's own rows and swaps that the per-score allowance permits, and it
rejects rows with a mistake planted into an oracle row (wrong order, a key
far below the boundary, a wrong score, a wrong count, a candidate from far
outside the candidate set)."""
from __future__ import annotations

import numpy as np

import oracle
import synthetic as syn
from tests import parity


def _case(mode, seed=5, S=256, H=1, D=32, top_k=16, g=8):
    q = syn.ar1_queries(S, H, D, seed, dtype="bf16")
    k = syn.pareto_keys(S, H, D, seed + 1, dtype="bf16")
    idx, sc = oracle.prefill(q, k, top_k, g, 2.0, mode)
    return q, k, idx, sc


def _check(q, k, idx_row, sc_row, ora_idx, ora_sc, i, mode, g=8, top_k=16):
    h = 0
    j = i // g
    n = max(j * g, 1)
    kv = parity.key_values(k, h, 0, n)
    proxy = oracle.proxy(q, g, h, j).astype(np.float64)
    cand = None
    if mode == "refine":
        cand, _ = oracle.prefill_candidates(q, k, h, j, top_k, g, 2.0)
        avec = parity.exact_ref.values(q[i, h])
    else:
        avec = proxy
    return parity.row_match(idx_row, sc_row, ora_idx, ora_sc, avec, kv, proxy=proxy, cand_idx=cand)


def test_oracle_rows_pass():
    for mode in ("refine", "reuse"):
        q, k, idx, sc = _case(mode)
        for i in range(8, 256, 13):
            assert _check(q, k, idx[i, 0], sc[i, 0], idx[i, 0], sc[i, 0], i, mode) is None


def test_planted_order_swap_is_caught():
    q, k, idx, sc = _case("refine")
    i = 200
    row = idx[i, 0].copy()
    row[[0, 5]] = row[[5, 0]]
    err = _check(q, k, row, None, idx[i, 0], sc[i, 0], i, "refine")
    assert err and "order" in err


def test_planted_far_key_is_caught():
    for mode in ("refine", "reuse"):
        q, k, idx, sc = _case(mode)
        i = 180
        row = idx[i, 0].copy()
        n = (i // 8) * 8
        # the prefix key with the lowest exact score under the ranking vector
        kv = parity.key_values(k, 0, 0, n)
        a = parity.exact_ref.values(q[i, 0]) if mode == "refine" else oracle.proxy(q, 8, 0, i // 8).astype(np.float64)
        worst = int(np.argmin(kv @ a))
        assert worst not in row
        row[-1] = worst
        err = _check(q, k, row, None, idx[i, 0], sc[i, 0], i, mode)
        assert err, mode


def test_planted_score_error_is_caught():
    q, k, idx, sc = _case("reuse")
    i = 150
    s = sc[i, 0].copy()
    s[3] *= np.float32(1.01)
    err = _check(q, k, idx[i, 0], s, idx[i, 0], sc[i, 0], i, "reuse")
    assert err and "score" in err


def test_planted_count_error_is_caught():
    q, k, idx, sc = _case("reuse")
    i = 150
    row = idx[i, 0].copy()
    row[-1] = -1
    err = _check(q, k, row, None, idx[i, 0], sc[i, 0], i, "reuse")
    assert err and "valid count" in err


def test_near_tie_swap_at_the_boundary_is_accepted():
    """Two keys whose exact scores differ by far less than their allowance
    may trade places across the row boundary."""
    D = 16
    S, g, top_k = 32, 8, 4
    q = np.zeros((S, 1, D), np.float32)
    q[:, 0, 0] = 1.0                       # ranking vector e_0 (for every group)
    k = np.zeros((S, 1, D), np.float32)
    # keys 0..7 score 10, 9, 8, 7 (boundary), then 7 + 2^-20 (k = 4), 1, ...
    vals = [10.0, 9.0, 8.0, 7.0, 7.0 + 2.0 ** -20, 1.0, 0.5, 0.25]
    k[:8, 0, 0] = vals
    k[:8, 0, 1] = 1.0                      # magnitude floor: A / sqrt(D) > 0
    idx, sc = oracle.prefill(q, k, top_k, g, 2.0, "reuse")
    i = 8
    np.testing.assert_array_equal(idx[i, 0], [0, 1, 2, 4])
    swapped = np.array([0, 1, 2, 3], np.int32)
    assert _check(q, k, swapped, None, idx[i, 0], sc[i, 0], i, "reuse", top_k=top_k) is None
    far = np.array([0, 1, 2, 5], np.int32)
    assert _check(q, k, far, None, idx[i, 0], sc[i, 0], i, "reuse", top_k=top_k)


def test_candidate_boundary_flip_needs_a_proxy_witness():
    """Refine: a key outside the oracle's candidate set may enter a GPU row
    only when its proxy score nearly ties some candidate's."""
    D = 16
    S, g, top_k = 32, 8, 2          # K = 4
    q = np.zeros((S, 1, D), np.float32)
    # group 1 (positions 8..15): proxy = e_0; member 8 ranks by e_1
    q[8:16, 0, 0] = 1.0
    q[8, 0, 1] = 8.0
    q[9, 0, 1] = -8.0   # the group mean of dim 1 stays 0
    k = np.zeros((S, 1, D), np.float32)
    # proxy scores of keys 0..7: 10, 9, 8, 7 | 7 - 2^-20 (key 4), 1, 0.5, 0.25
    k[:8, 0, 0] = [10.0, 9.0, 8.0, 7.0, 7.0 - 2.0 ** -20, 1.0, 0.5, 0.25]
    # member 8's own scores favour keys 4 and 5 (outside C)
    k[:8, 0, 1] = [0.0, 0.0, 0.0, 0.0, 1.0, 1.0, 0.0, 0.0]
    idx, sc = oracle.prefill(q, k, top_k, g, 2.0, "refine")
    i = 8
    cand, _ = oracle.prefill_candidates(q, k, 0, 1, top_k, g, 2.0)
    np.testing.assert_array_equal(cand, [0, 1, 2, 3])
    ora = idx[i, 0]
    # a GPU whose proxy scores swapped keys 3 and 4 takes key 4 (score 8 + 7)
    near = np.array([4, 0], np.int32)
    assert _check(q, k, near, None, ora, sc[i, 0], i, "refine", top_k=top_k) is None
    # key 5 (proxy score 1) cannot have entered the candidate set
    far = np.array([5, 0], np.int32)
    assert _check(q, k, far, None, ora, sc[i, 0], i, "refine", top_k=top_k)
