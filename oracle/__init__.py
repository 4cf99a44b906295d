"""PIVOT indexer -- CPU oracle (Python wrapper over ``pivot_oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library and never calls it. The arithmetic lives in plain C
(``pivot_oracle.c``); this module only marshals numpy arrays.

Inputs are numpy arrays on the host: float32 arrays for fp32 data, uint16
arrays holding raw bf16 bits for bf16 data. Outputs are numpy arrays:
int32 indices (-1 padding) and float32 scores (-inf padding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pivot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
REFINE, REUSE, REFINE_LITERAL = 0, 1, 2
# "refine_literal": the per-position-rescan Refine of the pages' pivot_refine
# code (prefill only; prefill() and prefill_rows())
MODES = {"refine": REFINE, "reuse": REUSE, "refine_literal": REFINE_LITERAL}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = f"{_LIB_PATH}.tmp{os.getpid()}"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    ci = ctypes.c_int
    lib.oracle_candidate_count.argtypes = [i32, f64]
    lib.oracle_candidate_count.restype = i64
    lib.oracle_proxy.argtypes = [vp, ci, i64, i32, i32, i32, i32, i64, vp]
    lib.oracle_proxy.restype = ci
    lib.oracle_prefill.argtypes = [vp, vp, ci, i64, i32, i32, i32, i32, f64, ci, i32, i32, vp, vp]
    lib.oracle_prefill.restype = ci
    lib.oracle_prefill_rows.argtypes = [vp, vp, ci, i64, i32, i32, i32, i32, f64, ci, i64, vp, vp, vp, vp]
    lib.oracle_prefill_rows.restype = ci
    lib.oracle_prefill_groups.argtypes = [vp, vp, ci, i64, i32, i32, i32, i32, f64, ci, i64, vp, vp, vp, vp]
    lib.oracle_prefill_groups.restype = ci
    lib.oracle_prefill_candidates.argtypes = [vp, vp, ci, i64, i32, i32, i32, i32, f64, i32, i64, vp, vp]
    lib.oracle_prefill_candidates.restype = i64
    lib.oracle_dense.argtypes = [vp, vp, ci, i64, i32, i32, i32, i32, i32, vp, vp]
    lib.oracle_dense.restype = ci
    lib.oracle_dense_rows.argtypes = [vp, vp, ci, i64, i32, i32, i32, i64, vp, vp, vp, vp]
    lib.oracle_dense_rows.restype = ci
    lib.oracle_decode.argtypes = [vp, vp, ci, vp, i32, i32, i32, i32, i32, f64, ci, i32, i32, vp, vp]
    lib.oracle_decode.restype = ci
    lib.oracle_decode_candidates.argtypes = [vp, vp, ci, vp, i32, i32, i32, i32, i32, f64, i32, i32, vp, vp]
    lib.oracle_decode_candidates.restype = i64
    lib.oracle_sparse_attention.argtypes = [vp, vp, vp, ci, i64, i32, i32, vp, i32, f64, vp]
    lib.oracle_sparse_attention.restype = ci
    lib.oracle_sparse_attention_rows.argtypes = [vp, vp, vp, ci, i64, i32, i32, vp, i32, i64, vp, vp, f64, vp]
    lib.oracle_sparse_attention_rows.restype = ci
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(q: np.ndarray, k: np.ndarray):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    if q.ndim != 3 or k.ndim != 3 or q.shape[1:] != k.shape[1:]:
        raise ValueError("q, k must be (rows, H, D) with equal H, D")
    return q, k, _dtype_code(q)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def candidate_count(top_k: int, candidate_ratio: float) -> int:
    """K = int(top_k * candidate_ratio); -1 when K < top_k."""
    return int(_load().oracle_candidate_count(top_k, candidate_ratio))


def proxy(q: np.ndarray, g: int, h: int, j: int) -> np.ndarray:
    """Proxy query (float32 values) of group j, head h."""
    q = np.ascontiguousarray(q)
    S, H, D = q.shape
    out = np.empty(D, np.float32)
    _check(_load().oracle_proxy(_ptr(q), _dtype_code(q), S, H, D, g, h, j, _ptr(out)), "oracle_proxy")
    return out


def prefill(q, k, top_k=64, g=8, candidate_ratio=2.0, mode="refine", heads=None):
    """Full prefill indexer. Returns (idx (S,H,top_k) int32, score float32).
    ``heads`` = (h_begin, h_end) limits the work; other heads stay -1/-inf."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    hb, he = heads if heads is not None else (0, H)
    idx = np.full((S, H, top_k), -1, np.int32)
    sc = np.full((S, H, top_k), -np.inf, np.float32)
    _check(_load().oracle_prefill(_ptr(q), _ptr(k), dt, S, H, D, top_k, g, candidate_ratio,
                                  MODES[mode], hb, he, _ptr(idx), _ptr(sc)), "oracle_prefill")
    return idx, sc


def prefill_rows(q, k, rows_i, rows_h, top_k=64, g=8, candidate_ratio=2.0, mode="refine"):
    """Indexer rows for selected (position, head) pairs: (n_rows, top_k)."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    ri = np.ascontiguousarray(rows_i, np.int64)
    rh = np.ascontiguousarray(rows_h, np.int32)
    n = ri.shape[0]
    idx = np.empty((n, top_k), np.int32)
    sc = np.empty((n, top_k), np.float32)
    _check(_load().oracle_prefill_rows(_ptr(q), _ptr(k), dt, S, H, D, top_k, g, candidate_ratio,
                                       MODES[mode], n, _ptr(ri), _ptr(rh), _ptr(idx), _ptr(sc)),
           "oracle_prefill_rows")
    return idx, sc


def prefill_groups(q, k, heads, groups, top_k=64, g=8, candidate_ratio=2.0, mode="refine"):
    """Whole groups (head heads[t], group groups[t]): (n, g, top_k) rows of
    all members, each group computed once."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    hh = np.ascontiguousarray(heads, np.int32)
    gg = np.ascontiguousarray(groups, np.int64)
    n = hh.shape[0]
    idx = np.empty((n, g, top_k), np.int32)
    sc = np.empty((n, g, top_k), np.float32)
    _check(_load().oracle_prefill_groups(_ptr(q), _ptr(k), dt, S, H, D, top_k, g, candidate_ratio,
                                         MODES[mode], n, _ptr(hh), _ptr(gg), _ptr(idx), _ptr(sc)),
           "oracle_prefill_groups")
    return idx, sc


def prefill_candidates(q, k, h, j, top_k=64, g=8, candidate_ratio=2.0):
    """Candidate set C (in total order) of group j, head h, with proxy scores."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    K = candidate_count(top_k, candidate_ratio)
    cand = np.empty(max(K, 1), np.int32)
    sc = np.empty(max(K, 1), np.float32)
    n = _load().oracle_prefill_candidates(_ptr(q), _ptr(k), dt, S, H, D, top_k, g, candidate_ratio,
                                          h, j, _ptr(cand), _ptr(sc))
    if n < 0:
        raise RuntimeError(f"oracle_prefill_candidates failed with code {n}")
    return cand[:n].copy(), sc[:n].copy()


def dense(q, k, top_k=64, heads=None):
    """Dense indexer: (S,H,top_k) int32 indices and float32 scores."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    hb, he = heads if heads is not None else (0, H)
    idx = np.full((S, H, top_k), -1, np.int32)
    sc = np.full((S, H, top_k), -np.inf, np.float32)
    _check(_load().oracle_dense(_ptr(q), _ptr(k), dt, S, H, D, top_k, hb, he, _ptr(idx), _ptr(sc)),
           "oracle_dense")
    return idx, sc


def dense_rows(q, k, rows_i, rows_h, top_k=64):
    """Dense indexer rows for selected (position, head) pairs: (n_rows, top_k)."""
    q, k, dt = _prep(q, k)
    S, H, D = q.shape
    ri = np.ascontiguousarray(rows_i, np.int64)
    rh = np.ascontiguousarray(rows_h, np.int32)
    n = ri.shape[0]
    idx = np.empty((n, top_k), np.int32)
    sc = np.empty((n, top_k), np.float32)
    _check(_load().oracle_dense_rows(_ptr(q), _ptr(k), dt, S, H, D, top_k, n, _ptr(ri), _ptr(rh),
                                     _ptr(idx), _ptr(sc)), "oracle_dense_rows")
    return idx, sc


def decode(q, k_cache, ctx_lens, g, top_k=64, candidate_ratio=2.0, mode="refine", heads=None):
    """Decode indexer: q (B*g,H,D), k_cache (sum ctx,H,D) -> (B*g,H,top_k)."""
    q = np.ascontiguousarray(q)
    kc = np.ascontiguousarray(k_cache)
    if q.dtype != kc.dtype:
        raise TypeError("q and k_cache must share a dtype")
    dt = _dtype_code(q)
    ctx = np.ascontiguousarray(ctx_lens, np.int64)
    B = ctx.shape[0]
    rows, H, D = q.shape
    if rows != B * g or kc.shape[1:] != (H, D) or kc.shape[0] != int(ctx.sum()):
        raise ValueError("decode shapes do not match (B*g, H, D) / (sum ctx, H, D)")
    hb, he = heads if heads is not None else (0, H)
    idx = np.full((rows, H, top_k), -1, np.int32)
    sc = np.full((rows, H, top_k), -np.inf, np.float32)
    _check(_load().oracle_decode(_ptr(q), _ptr(kc), dt, _ptr(ctx), B, g, H, D, top_k,
                                 candidate_ratio, MODES[mode], hb, he, _ptr(idx), _ptr(sc)),
           "oracle_decode")
    return idx, sc


def decode_candidates(q, k_cache, ctx_lens, g, h, b, top_k=64, candidate_ratio=2.0):
    """Candidate set C (in total order, indices relative to the sequence) of
    sequence b, head h of a decode step, with its proxy scores."""
    q = np.ascontiguousarray(q)
    kc = np.ascontiguousarray(k_cache)
    if q.dtype != kc.dtype:
        raise TypeError("q and k_cache must share a dtype")
    ctx = np.ascontiguousarray(ctx_lens, np.int64)
    B = ctx.shape[0]
    rows, H, D = q.shape
    K = candidate_count(top_k, candidate_ratio)
    cand = np.empty(max(K, 1), np.int32)
    sc = np.empty(max(K, 1), np.float32)
    n = _load().oracle_decode_candidates(_ptr(q), _ptr(kc), _dtype_code(q), _ptr(ctx), B, g, H, D, top_k,
                                         candidate_ratio, h, b, _ptr(cand), _ptr(sc))
    if n < 0:
        raise RuntimeError(f"oracle_decode_candidates failed with code {n}")
    return cand[:n].copy(), sc[:n].copy()


def sparse_attention(q, k, v, idx, scale=None):
    """Downstream sparse attention over the indices: (S, H, D) float32.
    scale defaults to D**-0.5 (the pages' demo)."""
    q, k, dt = _prep(q, k)
    v = np.ascontiguousarray(v)
    if v.dtype != q.dtype or v.shape != q.shape:
        raise ValueError("v must match q and k")
    idx = np.ascontiguousarray(idx, np.int32)
    S, H, D = q.shape
    if idx.ndim != 3 or idx.shape[:2] != (S, H):
        raise ValueError("idx must be (S, H, top_k)")
    out = np.empty((S, H, D), np.float32)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    _check(_load().oracle_sparse_attention(_ptr(q), _ptr(k), _ptr(v), dt, S, H, D, _ptr(idx), idx.shape[2],
                                           sc, _ptr(out)), "oracle_sparse_attention")
    return out


def sparse_attention_rows(q, k, v, idx_rows, rows_i, rows_h, scale=None):
    """Sparse attention of selected (position, head) rows with their index
    rows idx_rows (n_rows, top_k): (n_rows, D) float32."""
    q, k, dt = _prep(q, k)
    v = np.ascontiguousarray(v)
    if v.dtype != q.dtype or v.shape != q.shape:
        raise ValueError("v must match q and k")
    S, H, D = q.shape
    ir = np.ascontiguousarray(idx_rows, np.int32)
    ri = np.ascontiguousarray(rows_i, np.int64)
    rh = np.ascontiguousarray(rows_h, np.int32)
    out = np.empty((ri.shape[0], D), np.float32)
    sc = float(D) ** -0.5 if scale is None else float(scale)
    _check(_load().oracle_sparse_attention_rows(_ptr(q), _ptr(k), _ptr(v), dt, S, H, D, _ptr(ir), ir.shape[1],
                                                ri.shape[0], _ptr(ri), _ptr(rh), sc, _ptr(out)),
           "oracle_sparse_attention_rows")
    return out
