"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Bit-exact comparison is used where every float32 score is exact (small
integer inputs). Elsewhere rows are compared tie-tolerantly: float32
accumulation order may legitimately swap keys whose exact scores lie close
together.

Every tolerance below is derived from one per-score allowance. The GPU's
float32 score of key c against vector a may differ from the exact dot product
sigma_c by at most

    e_c = REL_TOL * max(|sigma_c|, A_c / sqrt(D)),   A_c = sum_d |a_d k_cd|,

the score rule of the comparison (1e-3 relative, with a floor against
cancellation near zero). A float32 dot product of D terms is off by at most
about D * 2^-24 * A_c (<= 7.7e-6 A_c at D = 128), far inside e_c. From this
allowance alone:

  * order: the GPU puts x before y only if sigma_x + e_x >= sigma_y - e_y, so
    along a GPU row exact scores may rise by at most e_x + e_y;
  * sets: a GPU entry x outside the oracle's row displaced some oracle entry
    y, so sigma_x >= sigma_y - e_x - e_y >= s_k - e_x - e_y (s_k the oracle's
    boundary score), and symmetrically for the oracle entries it lacks;
  * Refine candidate boundary: the GPU's candidate set may hold a key x
    outside the oracle's set C only if some y in C ranks below x in the GPU's
    proxy scores, i.e. sigma'_y - sigma'_x <= e'_x + e'_y (primed: proxy
    scores); it may lack a key y of C only if some z outside C (in the
    prefix) ranks above y there: sigma'_y - sigma'_z <= e'_y + e'_z. A Refine
    row that lost f of the oracle row's keys this way takes the next f keys
    of its candidate set, so its boundary moves down to the (nv + f)-th
    exact score over C.
"""
from __future__ import annotations

import numpy as np

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


class PrefixKeys:
    """float64 values of head h's keys kbase .. kbase+n-1 of a raw host key
    tensor (n, H, D), converted on demand: kv[cand] gives the rows of the
    prefix-relative indices cand."""

    def __init__(self, keys: np.ndarray, h: int, kbase: int, n: int):
        self.keys, self.h, self.kbase = keys, h, kbase
        self.shape = (n, keys.shape[2])

    def __getitem__(self, cand):
        return exact_ref.values(self.keys[self.kbase + np.asarray(cand, np.int64), self.h, :])


def structure_ok_device(idx, valid, limit, sc=None, chunk: int = 1 << 15):
    """structure_ok for large device outputs, vectorised with torch on the
    rows of idx (R, top_k): valid entries first then -1, exactly valid[r] of
    them, each below limit[r], distinct; with scores (R, top_k), non-increasing
    along the row with ascending index on equal scores and -inf padding.
    valid and limit are int64 device tensors of R entries."""
    import torch
    R, k = idx.shape
    pos = torch.arange(k, device=idx.device)
    for r0 in range(0, R, chunk):
        x = idx[r0:r0 + chunk].long()
        v = valid[r0:r0 + chunk, None]
        L = limit[r0:r0 + chunk, None]
        isv = pos[None, :] < v
        assert bool(torch.equal(x >= 0, isv)), f"rows {r0}..: valid count or padding"
        assert bool((x[~isv] == -1).all()), f"rows {r0}..: padding value"
        assert bool((x < L).all()), f"rows {r0}..: causality"
        u, _ = torch.sort(torch.where(isv, x, (1 << 40) + pos[None, :]), dim=1)
        assert bool((u[:, 1:] != u[:, :-1]).all()), f"rows {r0}..: duplicates"
        if sc is not None:
            s = sc[r0:r0 + chunk]
            both = isv[:, 1:]
            ok = (s[:, :-1] > s[:, 1:]) | ((s[:, :-1] == s[:, 1:]) & (x[:, :-1] < x[:, 1:]))
            assert bool((ok | ~both).all()), f"rows {r0}..: order"
            assert bool(torch.isneginf(s[~isv]).all()), f"rows {r0}..: score padding"


def key_values(keys: np.ndarray, h: int, kbase: int = 0, n: int | None = None) -> np.ndarray:
    """float64 values (exact) of head h's keys kbase .. kbase+n-1, shape (n, D)."""
    stop = keys.shape[0] if n is None else kbase + n
    return exact_ref.values(keys[kbase:stop, h, :])


def _scores(kv: np.ndarray, a: np.ndarray, cand: np.ndarray):
    """Exact scores, allowances e_c and magnitudes of keys `cand` against a."""
    if len(cand) == 0:
        z = np.zeros(0)
        return z, z
    rows = kv[cand]
    s = rows @ a
    mag = np.abs(rows) @ np.abs(a)
    return s, REL_TOL * np.maximum(np.abs(s), mag / np.sqrt(a.shape[0]))


def row_match(gpu_idx, gpu_sc, ora_idx, ora_sc, avec, kv, *, proxy=None, cand_idx=None):
    """Tie-tolerant check of one row; returns an error string or None.

    gpu_idx / ora_idx: the row (indices, -1 padding) of the GPU and the
    oracle; gpu_sc: the GPU's scores (or None); ora_sc: the oracle's scores;
    avec: float64 vector that ranks the row (the query for Refine and dense,
    the proxy for Reuse); kv: float64 key values of the row's whole prefix
    (key c at kv[c]). For Refine rows also proxy (float64) and cand_idx, the
    oracle's candidate set C.
    """
    nv = int((ora_idx >= 0).sum())
    if int((gpu_idx >= 0).sum()) != nv:
        return f"valid count {int((gpu_idx >= 0).sum())} != {nv}"
    if nv == 0:
        return None
    g = gpu_idx[:nv].astype(np.int64)
    o = ora_idx[:nv].astype(np.int64)
    if (g < 0).any() or (g >= kv.shape[0]).any():
        return "index outside the prefix"
    s_g, e_g = _scores(kv, avec, g)
    # scores: each returned slot's score within its allowance
    if gpu_sc is not None:
        bad = np.abs(gpu_sc[:nv].astype(np.float64) - s_g) > e_g
        if bad.any():
            return f"score mismatch at slots {np.nonzero(bad)[0][:5]}"
    # order: exact scores along the GPU row non-increasing within e_x + e_y
    rise = s_g[1:] - s_g[:-1]
    bad = rise > e_g[1:] + e_g[:-1]
    if bad.any():
        return f"order: exact scores rise beyond tolerance after slots {np.nonzero(bad)[0][:5]}"
    extra = np.setdiff1d(g, o)
    missing = np.setdiff1d(o, g)
    if len(extra) == 0 and len(missing) == 0:
        return None
    s_o, _ = _scores(kv, avec, o[nv - 1:nv])
    sk = float(s_o[0])
    s_e, e_e = _scores(kv, avec, extra)
    s_m, e_m = _scores(kv, avec, missing)
    E_m = float(e_m.max()) if len(e_m) else 0.0
    E_e = float(e_e.max()) if len(e_e) else 0.0
    ok_e = s_e >= sk - e_e - E_m
    ok_m = s_m <= sk + e_m + E_e
    if cand_idx is not None:
        cand_idx = np.asarray(cand_idx, np.int64)
        sp_c, ep_c = _scores(kv, proxy, cand_idx)
        # flips into the candidate set: a witness y in C the GPU ranked below
        out_c = ~np.isin(extra, cand_idx)
        if out_c.any():
            sp_x, ep_x = _scores(kv, proxy, extra[out_c])
            wit = (sp_c[None, :] - sp_x[:, None]) <= (ep_x[:, None] + ep_c[None, :])
            flip_in = np.zeros(len(extra), bool)
            flip_in[np.nonzero(out_c)[0]] = wit.any(axis=1)
            ok_e |= flip_in
        # flips out of it: a witness z outside C (in the prefix) ranked above
        in_c = np.isin(missing, cand_idx) & ~ok_m
        n_fo = 0
        if in_c.any():
            others = np.setdiff1d(np.arange(kv.shape[0]), cand_idx)
            sp_z, ep_z = _scores(kv, proxy, others)
            sp_y, ep_y = _scores(kv, proxy, missing[in_c])
            flip_out = np.zeros(len(missing), bool)
            if len(others):
                wit = np.zeros(len(sp_y), bool)
                for t in range(len(sp_y)):
                    wit[t] = ((sp_y[t] - sp_z) <= (ep_y[t] + ep_z)).any()
                flip_out[np.nonzero(in_c)[0]] = wit
            ok_m |= flip_out
            n_fo = int(flip_out.sum())
        if n_fo:
            # the row's boundary moves down to the (nv + n_fo)-th score over C
            s_c, _ = _scores(kv, avec, cand_idx)
            s_c = np.sort(s_c)[::-1]
            s_ext = float(s_c[min(nv + n_fo, len(s_c)) - 1])
            ok_e |= np.isin(extra, cand_idx) & (s_e >= s_ext - e_e - E_m)
    if not ok_e.all() or not ok_m.all():
        return (f"set differs beyond tolerance: extra {extra[~ok_e][:5]} missing {missing[~ok_m][:5]} "
                f"(boundary {sk})")
    return None


def tolerant_row_match(gpu_idx, gpu_sc, ora_idx, ora_sc, avec, keys, h, D, kbase=0,
                       cand_idx=None, cand_sc=None, proxy=None, n_prefix=None, kv=None):
    """row_match on raw host keys (head h, prefix starting at kbase). The
    prefix is n_prefix keys long (default: every key from kbase on); kv, when
    given, is the float64 prefix already converted."""
    del D, cand_sc
    if kv is None:
        kv = key_values(keys, h, kbase, n_prefix)
    return row_match(gpu_idx, gpu_sc, ora_idx, ora_sc, avec, kv, proxy=proxy, cand_idx=cand_idx)
