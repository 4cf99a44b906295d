"""Runs oracle calls over the host's cores.

TEST INFRASTRUCTURE, like the rest of this package: used by the tests and by
the CPU-baseline leg of the benchmark only. It holds no arithmetic of the
method; it only distributes calls of ``oracle`` functions over processes.

The oracle is single-threaded C; full-size parity runs many independent
calls (one per head, or per group, or per sequence) in worker processes.
Workers are started with "spawn" (nothing of the parent's GPU state is
inherited) and read the input arrays from .npy files that they memory-map,
so a multi-gigabyte key tensor is written once and shared through the page
cache instead of being pickled per task.

    with OraclePool() as pool:
        q_ref = pool.put(q_head)              # array -> shared file
        res = pool.map([("prefill", dict(q=q_ref, k=k_ref, top_k=512, ...)), ...])

A task is (name of an ``oracle`` function, keyword arguments); ``Shared``
arguments are replaced by the memory-mapped array in the worker.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np


class Shared:
    """A handle to an array written to the pool's directory (rows start ..
    stop of it when sliced)."""

    def __init__(self, path: str, start: int | None = None, stop: int | None = None):
        self.path = path
        self.start = start
        self.stop = stop

    def rows(self, start: int, stop: int) -> "Shared":
        return Shared(self.path, start, stop)

    def load(self) -> np.ndarray:
        a = np.load(self.path, mmap_mode="r")
        return a if self.start is None else a[self.start:self.stop]


def workers_default() -> int:
    # one GPU's share of the machine's host cores, at most 16
    return max(1, min(16, os.cpu_count() or 1))


def prefill_groups_of_head(q, k, groups, top_k, g, candidate_ratio, mode):
    """Whole groups of a one-head prefill (q, k shaped (S, 1, D)): their rows
    (n, g, top_k), and per group the proxy and, for Refine, the candidate
    set C in total order."""
    import oracle
    groups = np.asarray(groups, np.int64)
    idx, sc = oracle.prefill_groups(q, k, np.zeros(len(groups), np.int32), groups, top_k, g, candidate_ratio,
                                    mode)
    proxies = [oracle.proxy(q, g, 0, int(j)) for j in groups]
    cands = None
    if mode == "refine":
        cands = [oracle.prefill_candidates(q, k, 0, int(j), top_k, g, candidate_ratio)[0] for j in groups]
    return idx, sc, proxies, cands


def decode_sequence(q, kc, ctx, g, top_k, candidate_ratio, mode):
    """One sequence of one head (q (g, 1, D), kc (ctx, 1, D)): its g rows,
    the proxy and, for Refine, the candidate set."""
    import oracle
    lens = np.array([ctx], np.int64)
    idx, sc = oracle.decode(q, kc, lens, g, top_k, candidate_ratio, mode)
    cand = oracle.decode_candidates(q, kc, lens, g, 0, 0, top_k, candidate_ratio)[0] if mode == "refine" else None
    return idx[:, 0], sc[:, 0], oracle.proxy(q, g, 0, 0), cand


def timed_groups(q, k, seconds, seed, top_k, g, candidate_ratio, mode):
    """Whole groups drawn uniformly over (head, group) and run one after the
    other until `seconds` have passed; returns (rows, groups, seconds)."""
    import time

    import oracle
    S, H = q.shape[0], q.shape[1]
    G = (S + g - 1) // g
    rng = np.random.default_rng(seed)
    rows = groups = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        hh = rng.integers(0, H, 1).astype(np.int32)
        jj = rng.integers(0, G, 1)
        oracle.prefill_groups(q, k, hh, jj, top_k, g, candidate_ratio, mode)
        rows += int(min(g, S - jj[0] * g))
        groups += 1
    return rows, groups, time.perf_counter() - t0


_TASKS = {"prefill_groups_of_head": prefill_groups_of_head, "decode_sequence": decode_sequence,
          "timed_groups": timed_groups}


def _run(task):
    name, kwargs = task
    import oracle
    args = {k: (v.load() if isinstance(v, Shared) else v) for k, v in kwargs.items()}
    fn = _TASKS[name] if name in _TASKS else getattr(oracle, name)
    return fn(**args)


class OraclePool:
    def __init__(self, workers: int | None = None, need_bytes: int = 0):
        self.workers = workers or workers_default()
        self.need = need_bytes
        self.dir = None
        self.pool = None
        self.n = 0

    def __enter__(self):
        base = None  # the default temporary directory (its files stay in the page cache)
        try:
            st = os.statvfs("/dev/shm")
            if os.access("/dev/shm", os.W_OK) and st.f_bavail * st.f_frsize > 2 * self.need + (1 << 30):
                base = "/dev/shm"
        except OSError:
            pass
        import oracle
        oracle._load()  # (re)built here once, not by every worker at the same time
        self.dir = tempfile.mkdtemp(prefix="oracle_pool_", dir=base)
        self.pool = mp.get_context("spawn").Pool(self.workers)
        return self

    def put(self, a: np.ndarray) -> Shared:
        path = os.path.join(self.dir, f"a{self.n}.npy")
        self.n += 1
        np.save(path, np.ascontiguousarray(a))
        return Shared(path)

    def drop(self, ref: Shared):
        os.unlink(ref.path)

    def map(self, tasks):
        return self.pool.map(_run, tasks, chunksize=1)

    def __exit__(self, *exc):
        try:
            self.pool.close()
            self.pool.join()
        finally:
            shutil.rmtree(self.dir, ignore_errors=True)
        return False
