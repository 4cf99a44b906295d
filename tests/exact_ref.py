"""Exact-arithmetic brute force used to pin the oracle on tiny inputs.

Written independently of ``oracle/`` in exact rational arithmetic
(``fractions.Fraction``) with Python's ``sorted`` as the selection: a proxy is
the exact mean rounded to the input type with a round-to-nearest-even written
from its definition; a score is the exact dot product rounded once to float32.
Too slow for anything but tiny cases, which is what it is for.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def rne(x: Fraction, mant_bits: int) -> Fraction:
    """Round x to the nearest value with `mant_bits` significant bits, ties to
    even (normal range only; exact zero stays zero)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - mant_bits + 1)
    scaled = a / ulp
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def to_f32(x: Fraction) -> float:
    return float(rne(x, 24))


def values(a: np.ndarray) -> np.ndarray:
    """Host input (float32 or uint16 bf16 bits) -> float64 values (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def proxy_exact(qv: np.ndarray, i0: int, m: int, h: int, bf16: bool) -> list[Fraction]:
    """Mean of rows i0..i0+m-1 of head h, rounded as the pages' dtype rules
    say: float32 sum (exact here for small integers), float32 division, then
    bf16 for bf16 inputs. Inputs are small integers, so the float32 sum is
    exact and the single float32 rounding of sum/m is the only rounding."""
    D = qv.shape[2]
    out = []
    for d in range(D):
        s = sum(Fraction(float(qv[i, h, d])) for i in range(i0, i0 + m))
        v = rne(s / m, 24)
        if bf16:
            v = rne(v, 8)
        out.append(v)
    return out


def dot_f32(a: list[Fraction], kv: np.ndarray, c: int, h: int) -> float:
    s = sum(a[d] * Fraction(float(kv[c, h, d])) for d in range(kv.shape[2]))
    v = to_f32(s)
    return 0.0 if v == 0.0 else v


def topk_exact(scored: list[tuple[float, int]], k: int) -> list[tuple[float, int]]:
    return sorted(scored, key=lambda t: (-t[0], t[1]))[:k]


def pivot_exact(q: np.ndarray, k: np.ndarray, top_k: int, g: int, K: int, mode: str):
    """(S, H, top_k) indices and scores by exact arithmetic."""
    bf16 = q.dtype == np.uint16
    qv, kv = values(q), values(k)
    S, H, D = q.shape
    idx = np.full((S, H, top_k), -1, np.int64)
    sc = np.full((S, H, top_k), -np.inf, np.float64)
    for h in range(H):
        for i0 in range(0, S, g):
            m = min(g, S - i0)
            n = max(i0, 1)
            p = proxy_exact(qv, i0, m, h, bf16)
            cand = topk_exact([(dot_f32(p, kv, c, h), c) for c in range(n)], K)
            for i in range(i0, i0 + m):
                if mode == "reuse":
                    row = cand[:top_k]
                else:
                    qi = [Fraction(float(x)) for x in qv[i, h]]
                    row = topk_exact([(dot_f32(qi, kv, c, h), c) for _, c in cand], top_k)
                for t, (s, c) in enumerate(row):
                    idx[i, h, t] = c
                    sc[i, h, t] = s
    return idx, sc


def dense_exact(q: np.ndarray, k: np.ndarray, top_k: int):
    qv, kv = values(q), values(k)
    S, H, D = q.shape
    idx = np.full((S, H, top_k), -1, np.int64)
    sc = np.full((S, H, top_k), -np.inf, np.float64)
    for h in range(H):
        for i in range(S):
            qi = [Fraction(float(x)) for x in qv[i, h]]
            row = topk_exact([(dot_f32(qi, kv, c, h), c) for c in range(max(i, 1))], top_k)
            for t, (s, c) in enumerate(row):
                idx[i, h, t] = c
                sc[i, h, t] = s
    return idx, sc


def literal_exact(q: np.ndarray, k: np.ndarray, top_k: int, g: int, K: int):
    """The literal per-position Refine by exact arithmetic: position i >= 1
    scans keys [0, i) with its group's proxy, keeps its own first min(K, i)
    and re-scores them with q_i; position 0 is all padding."""
    bf16 = q.dtype == np.uint16
    qv, kv = values(q), values(k)
    S, H, D = q.shape
    idx = np.full((S, H, top_k), -1, np.int64)
    sc = np.full((S, H, top_k), -np.inf, np.float64)
    for h in range(H):
        for i in range(1, S):
            i0 = (i // g) * g
            p = proxy_exact(qv, i0, min(g, S - i0), h, bf16)
            cand = topk_exact([(dot_f32(p, kv, c, h), c) for c in range(i)], K)
            qi = [Fraction(float(x)) for x in qv[i, h]]
            row = topk_exact([(dot_f32(qi, kv, c, h), c) for _, c in cand], top_k)
            for t, (s, c) in enumerate(row):
                idx[i, h, t] = c
                sc[i, h, t] = s
    return idx, sc
