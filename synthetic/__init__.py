"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the indexer: it only draws inputs. The
distributions model the two observations PIVOT builds on ("PIVOT Explained",
section "How It Works"): nearby queries overlap in their top-k selections
(AR(1) queries along the sequence) and indexer scores are long-tailed along
the key axis (keys with Pareto-distributed norms).

Every generator returns host numpy arrays: float32 values, or uint16 raw bf16
bits (round-to-nearest-even from the float32 draw) when ``dtype="bf16"``.
All draws come from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

import numpy as np


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def gaussian(shape, seed: int, dtype: str = "f32") -> np.ndarray:
    """i.i.d. N(0, 1) entries."""
    rng = np.random.default_rng(seed)
    return _finish(rng.standard_normal(shape, dtype=np.float32), dtype)


def integers(shape, seed: int, a: int, dtype: str = "f32") -> np.ndarray:
    """i.i.d. integers uniform in [-a, a] (exactly representable)."""
    rng = np.random.default_rng(seed)
    return _finish(rng.integers(-a, a + 1, size=shape).astype(np.float32), dtype)


def ar1_queries(S: int, H: int, D: int, seed: int, rho: float = 0.95, dtype: str = "bf16") -> np.ndarray:
    """AR(1) along the sequence, per (head, dim): q_0 = e_0 / sqrt(1 - rho^2),
    q_t = rho * q_{t-1} + e_t with e ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, H, D), dtype=np.float32)
    q[0] /= np.float32(np.sqrt(1.0 - rho * rho))
    r = np.float32(rho)
    # the recursion runs along the sequence, one vector step per position
    for t in range(1, S):
        q[t] += r * q[t - 1]
    return _finish(q, dtype)


def pareto_keys(S: int, H: int, D: int, seed: int, alpha: float = 2.0, dtype: str = "bf16") -> np.ndarray:
    """Keys k = r * z / |z| per (token, head): z ~ N(0, I_D) directions,
    r = (1 - U)^(-1/alpha) Pareto(x_m = 1, alpha) norms."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((S, H, D), dtype=np.float32)
    u = rng.random((S, H, 1), dtype=np.float64)
    r = (1.0 - u) ** (-1.0 / alpha)
    z /= np.linalg.norm(z, axis=2, keepdims=True)
    z *= r.astype(np.float32)
    return _finish(z, dtype)


def decode_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Context lengths uniform in [lo, hi] (int64)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


# ---------------------------------------------------------------- workloads
# The five workloads the indexer is measured and checked on. Seeds: 1000 + c,
# and 1100 + c for an integer-valued twin.

def tiny_prefill(integer: bool = False):
    """S=1024, H=8, D=64 fp32; N(0,1), or integers in [-8, 8]; top_k=64,
    g=8, K=128."""
    S, H, D = 1024, 8, 64
    if integer:
        q = integers((S, H, D), 1101, 8, "f32")
        k = integers((S, H, D), 2101, 8, "f32")
    else:
        q = gaussian((S, H, D), 1001, "f32")
        k = gaussian((S, H, D), 2001, "f32")
    return dict(q=q, k=k, top_k=64, g=8, candidate_ratio=2.0)


def int_prefill():
    """S=16384, H=16, D=128 bf16 integers in [-4, 4]; top_k=512, g=8, K=1024."""
    S, H, D = 16384, 16, 128
    q = integers((S, H, D), 1002, 4, "bf16")
    k = integers((S, H, D), 2002, 4, "bf16")
    return dict(q=q, k=k, top_k=512, g=8, candidate_ratio=2.0)


def long_prefill(S: int = 65536, H: int = 64, g: int = 8, seed: int = 1003):
    """AR(1) bf16 queries, Pareto-norm bf16 keys, D=128, top_k=2048, K=4096.
    Defaults: the S=65536, H=64, g=8 workload; (131072, 32, 16, 1004) is the
    long one."""
    D = 128
    q = ar1_queries(S, H, D, seed)
    k = pareto_keys(S, H, D, seed + 1000)
    return dict(q=q, k=k, top_k=2048, g=g, candidate_ratio=2.0)


def decode_step(g: int = 2, B: int = 64, H: int = 8, lo: int = 32768, hi: int = 131072, seed: int = 1005):
    """B sequences with contexts uniform in [lo, hi]; H=8, D=128 bf16
    Pareto-norm key cache (packed by sequence); g AR(1) MTP queries per
    sequence; top_k=2048, K=4096."""
    D = 128
    ctx = decode_lengths(B, lo, hi, seed)
    kc = pareto_keys(int(ctx.sum()), H, D, seed + 1000)
    qs = [ar1_queries(g, H, D, seed + 2000 + b, dtype="f32") for b in range(B)]
    q = to_bf16_bits(np.concatenate(qs, axis=0))
    return dict(q=q, k_cache=kc, ctx_lens=ctx, g=g, top_k=2048, candidate_ratio=2.0)


# ------------------------------------------------------------ device draws
# The long workloads are drawn on the device with torch's seeded generator
# (same distributions and recipe as above; different random streams). The
# AR(1) recursion runs blockwise in float64: inside a block of B steps,
#   q_{t0+u} = rho^u * (rho * q_{t0-1} + sum_{v<=u} rho^{-v} e_{t0+v}).

def ar1_queries_device(S: int, H: int, D: int, seed: int, device, rho: float = 0.95, block: int = 128):
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    e = torch.randn((S, H, D), generator=gen, device=device, dtype=torch.float32)
    out = torch.empty((S, H, D), device=device, dtype=torch.bfloat16)
    carry = e[0].double() / float(np.sqrt(1.0 - rho * rho))
    out[0] = carry.to(torch.bfloat16)
    u = torch.arange(block, device=device, dtype=torch.float64)
    pw = rho ** u
    ipw = rho ** (-u)
    t = 1
    while t < S:
        n = min(block, S - t)
        c = torch.cumsum(e[t:t + n].double() * ipw[:n, None, None], dim=0)
        blk = pw[:n, None, None] * (rho * carry + c)
        out[t:t + n] = blk.to(torch.bfloat16)
        carry = blk[-1]
        t += n
    return out


def pareto_keys_device(S: int, H: int, D: int, seed: int, device, alpha: float = 2.0, chunk: int = 1 << 16):
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty((S, H, D), device=device, dtype=torch.bfloat16)
    for s0 in range(0, S, chunk):
        n = min(chunk, S - s0)
        z = torch.randn((n, H, D), generator=gen, device=device, dtype=torch.float32)
        u = torch.rand((n, H, 1), generator=gen, device=device, dtype=torch.float64)
        r = ((1.0 - u) ** (-1.0 / alpha)).float()
        out[s0:s0 + n] = (z * (r / torch.linalg.vector_norm(z, dim=2, keepdim=True))).to(torch.bfloat16)
    return out


def long_prefill_device(device, S: int = 65536, H: int = 64, g: int = 8, seed: int = 1003):
    """Device tensors of the AR(1) / Pareto-norm prefill workload."""
    D = 128
    return dict(q=ar1_queries_device(S, H, D, seed, device), k=pareto_keys_device(S, H, D, seed + 1000, device),
                top_k=2048, g=g, candidate_ratio=2.0)


def decode_step_device(device, g: int = 2, B: int = 64, H: int = 8, lo: int = 32768, hi: int = 131072,
                       seed: int = 1005):
    """Device tensors of the decode workload: B sequences, contexts uniform
    in [lo, hi], Pareto-norm bf16 cache, g AR(1) queries per sequence."""
    import torch
    D = 128
    ctx = decode_lengths(B, lo, hi, seed)
    kc = pareto_keys_device(int(ctx.sum()), H, D, seed + 1000, device)
    q = torch.cat([ar1_queries_device(g, H, D, seed + 2000 + b, device) for b in range(B)], dim=0)
    return dict(q=q.contiguous(), k_cache=kc, ctx_lens=ctx, g=g, top_k=2048, candidate_ratio=2.0)


def bf16_tensor_to_bits(t) -> np.ndarray:
    """Host uint16 bf16 bits of a device bfloat16 tensor (for the oracle)."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
