"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Bit-exact comparison is used where every float32 score is exact (small
integer inputs). Elsewhere rows are compared tie-tolerantly: float32
accumulation order may legitimately swap keys whose exact scores are within
the tolerance of the row's boundary score.
"""
from __future__ import annotations

import numpy as np

import oracle
from tests import exact_ref

REL_TOL = 1e-3


def to_host(t):
    return t.detach().cpu().numpy()


def structure_ok(idx: np.ndarray, sc: np.ndarray | None, limits: np.ndarray, valid: np.ndarray):
    """Valid entries first then -1, distinct, below the row's prefix limit,
    exactly `valid` of them; scores non-increasing with index tie order."""
    rows = idx.reshape(-1, idx.shape[-1])
    lim = np.broadcast_to(limits, idx.shape[:-1]).reshape(-1)
    val = np.broadcast_to(valid, idx.shape[:-1]).reshape(-1)
    scr = None if sc is None else sc.reshape(-1, sc.shape[-1])
    for r in range(rows.shape[0]):
        row = rows[r]
        nv = int(val[r])
        assert (row[:nv] >= 0).all() and (row[nv:] == -1).all(), f"row {r}: padding"
        assert (row[:nv] < lim[r]).all(), f"row {r}: causality"
        assert len(np.unique(row[:nv])) == nv, f"row {r}: duplicates"
        if scr is not None:
            s = scr[r]
            assert np.isneginf(s[nv:]).all()
            ok = (s[:-1] > s[1:]) | ((s[:-1] == s[1:]) & (row[:-1] < row[1:]))
            assert ok[: max(nv - 1, 0)].all(), f"row {r}: order"


def exact_scores(avec: np.ndarray, keys: np.ndarray, h: int, cand: np.ndarray, kbase: int = 0):
    """float64 scores and |a|.|k| magnitudes of keys `cand` (head h)."""
    kv = exact_ref.values(keys[kbase + cand, h, :]) if len(cand) else np.zeros((0, avec.shape[0]))
    s = kv @ avec
    mag = np.abs(kv) @ np.abs(avec)
    return s, mag


def tolerant_row_match(gpu_idx, gpu_sc, ora_idx, ora_sc, avec, keys, h, D, kbase=0,
                       cand_idx=None, cand_sc=None, proxy=None):
    """Tie-tolerant check of one row; returns an error string or None.

    Scores of returned keys must match their exact values; the two sets may
    differ only by keys whose exact score lies within tolerance of the
    oracle's boundary score. For Refine rows (cand_* given) a key may also
    differ because it sits at the candidate-set boundary of the proxy scan.
    """
    nv = int((ora_idx >= 0).sum())
    if int((gpu_idx >= 0).sum()) != nv:
        return f"valid count {int((gpu_idx >= 0).sum())} != {nv}"
    if nv == 0:
        return None
    g = gpu_idx[:nv].astype(np.int64)
    o = ora_idx[:nv].astype(np.int64)
    s_g, m_g = exact_scores(avec, keys, h, g, kbase)
    tol_g = REL_TOL * np.maximum(np.abs(s_g), m_g / np.sqrt(D))
    if gpu_sc is not None:
        bad = np.abs(gpu_sc[:nv].astype(np.float64) - s_g) > tol_g
        if bad.any():
            return f"score mismatch at slots {np.nonzero(bad)[0][:5]}"
    sk = float(ora_sc[nv - 1])
    _, m_k = exact_scores(avec, keys, h, o[nv - 1:nv], kbase)
    tau = REL_TOL * max(abs(sk), float(m_k[0]) / np.sqrt(D), 1e-30)
    extra = np.setdiff1d(g, o)
    missing = np.setdiff1d(o, g)
    if len(extra) == 0 and len(missing) == 0:
        return None
    s_e, _ = exact_scores(avec, keys, h, extra, kbase)
    s_m, _ = exact_scores(avec, keys, h, missing, kbase)
    near_cand = None
    if cand_idx is not None:
        # proxy-boundary flips: keys whose proxy score is near the K-th
        pk = float(cand_sc[-1])
        ps_e, pm_e = exact_scores(proxy, keys, h, extra, kbase)
        ps_m, pm_m = exact_scores(proxy, keys, h, missing, kbase)
        tp_e = REL_TOL * np.maximum(np.abs(pk), pm_e / np.sqrt(D)) * 4
        tp_m = REL_TOL * np.maximum(np.abs(pk), pm_m / np.sqrt(D)) * 4
        in_c = np.isin(extra, cand_idx)
        near_cand = (~in_c & (ps_e >= pk - tp_e)), (np.isin(missing, cand_idx) & (ps_m <= pk + tp_m))
    ok_e = s_e >= sk - tau
    ok_m = s_m <= sk + tau
    if near_cand is not None:
        ok_e |= near_cand[0]
        ok_m |= near_cand[1]
    if not ok_e.all() or not ok_m.all():
        return (f"set differs beyond tolerance: extra {extra[~ok_e][:5]} missing {missing[~ok_m][:5]} "
                f"(boundary {sk}, tau {tau})")
    return None
