#!/usr/bin/env python3
"""Benchmark of the PIVOT indexer on one MI355X.

Workload (the metric's): prefill S=65536, H=64, D=128 bf16, AR(1) queries
(rho=0.95) and Pareto(alpha=2)-norm keys, top_k=2048, g=8, K=4096. A step is
one PIVOT-Refine prefill call (proxy, sample scan, thresholds, main scan,
candidate select, fallback, refine), inputs resident in HBM. The JSON line
also carries PIVOT-Reuse on the same inputs, the decode workload (64
sequences, contexts U[32768, 131072], H=8, g in {2, 4}), per-kernel times
from HIP events recorded on the library's stream, the roofline of the
dominant kernel, recall@top_k against the dense indexer on sampled rows and
the CPU oracle timed on this host.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, MI355X dense bf16 MFMA


def log(msg: str):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def prefix_sums(S: int, g: int, K: int):
    """Sum over groups of the prefix length n_j = max(j*g, 1) and of
    min(K, n_j)."""
    import numpy as np
    j = np.arange((S + g - 1) // g, dtype=np.int64)
    n = np.maximum(j * g, 1)
    return int(n.sum()), int(np.minimum(n, K).sum())


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_token_selection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def counted_traffic(stage: str, S: int, H: int, g: int):
    """HBM bytes per launch of a stage's kernel, as counted by FETCH_SIZE and
    WRITE_SIZE (scaled by a copy kernel of known size) in a committed counter
    summary; None when there is none for this workload or the kernel sources
    have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_hbm_traffic_S{S}_H{H}_g{g}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(" "):
                key, _, v = ln.partition(":")
                vals[key.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(vals["read_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recall_rows(a, b, skip_first_rows: int = 0, H: int = 1):
    """Recall@top_k of index rows a against reference rows b (device int32
    (S*H, top_k), -1 padding): mean over rows of |a & b| / |b|, leaving out
    the first skip_first_rows positions (position 0 has a single key)."""
    import torch
    k = b.shape[1]
    tot, n = 0.0, 0
    for r0 in range(skip_first_rows * H, b.shape[0], 1 << 16):
        bb, aa = b[r0:r0 + (1 << 16)].long(), a[r0:r0 + (1 << 16)].long()
        bs, _ = torch.sort(torch.where(bb >= 0, bb, 1 << 40), dim=1)
        pos = torch.searchsorted(bs, aa).clamp(max=k - 1)
        hit = ((torch.gather(bs, 1, pos) == aa) & (aa >= 0)).sum(1)
        nb = (bb >= 0).sum(1)
        ok = nb > 0
        tot += float((hit[ok].double() / nb[ok].double()).sum())
        n += int(ok.sum())
    return tot / max(n, 1)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def time_calls(fn, steps: int, warmup: int, pv):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    pv.profile_read()
    pv.profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = pv.profile_read()
    pv.profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    per_stage = {k: v[0] / steps for k, v in stages.items()}
    launches = {k: v[1] // steps for k, v in stages.items()}
    return ms, wall / steps * 1e3, per_stage, launches


def sweep(args, dev, torch, np, syn, pv):
    """Recall-speed grid over group size and candidate ratio (the pages fix g
    by hand and give no adaptive rule); one JSON line."""
    S, H, D = 65536, 64, 128
    log(f"drawing prefill S={S} H={H} D={D} on the device")
    cfg = syn.long_prefill_device(dev, S=S, H=H, g=8, seed=1003)
    q, k = cfg["q"], cfg["k"]
    rng = np.random.default_rng(17)
    nrows = 1024
    ri = torch.from_numpy(rng.integers(32, S, nrows)).to(dev)
    rh = torch.from_numpy(rng.integers(0, H, nrows)).to(dev)
    grid = []
    for top_k, ratios in ((2048, (1.0, 1.5, 2.0, 4.0)), (1024, (1.0, 1.5, 2.0, 4.0))):
        out = torch.empty((S, H, top_k), dtype=torch.int32, device=dev)
        dense_ms, _, _, _ = time_calls(lambda: pv.dense_index(q, k, top_k, out=out, max_workspace_bytes=48 << 30),
                                       1, 1, pv)
        ref = out[ri, rh].cpu().numpy()
        ref_sets = [set(r[r >= 0].tolist()) for r in ref]
        for g in (1, 2, 4, 8, 16, 32):
            for ratio in ratios:
                # Reuse takes the proxy's first top_k candidates whatever the
                # ratio: once per group size
                for mode in ("refine", "reuse") if ratio == ratios[0] else ("refine",):
                    # small groups need large workspaces: heads then run in chunks
                    def call():
                        pv.index_prefill(q, k, top_k, g, ratio, mode, out=out, max_workspace_bytes=200 << 30)
                    ms, _, _, _ = time_calls(call, max(1, args.steps // 2), 1, pv)
                    rows = out[ri, rh].cpu().numpy()
                    rec = float(np.mean([len(set(a[a >= 0].tolist()) & b) / len(b) for a, b in zip(rows, ref_sets)]))
                    e = {"top_k": top_k, "g": g, "candidate_ratio": ratio, "K": pv.candidate_count(top_k, ratio),
                         "mode": mode, "ms_per_call": ms, "queries_per_s": S * H / (ms / 1e3),
                         "speedup_vs_dense": dense_ms / ms, "recall": rec}
                    grid.append(e)
                    log(f"top_k={top_k} g={g:2d} ratio={ratio} {mode}: {ms:7.2f} ms, recall {rec:.4f}, "
                        f"x{dense_ms / ms:.2f} vs dense")
        grid.append({"top_k": top_k, "mode": "dense", "ms_per_call": dense_ms,
                     "queries_per_s": S * H / (dense_ms / 1e3)})
        del out
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "g x candidate_ratio", "workload": f"S={S} H={H} D={D} bf16 AR(1)/Pareto seed 1003",
                      "recall_rows": nrows, "recall_against": "dense indexer (GPU), seed 17 sample",
                      "grid": grid}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-reuse", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip timing the dense indexer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip timing the downstream sparse attention on the indexer's rows")
    ap.add_argument("--no-literal", action="store_true",
                    help="skip the literal per-position Refine comparison (8 heads of the S=65536 workload)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (tiny, S=16384 integer, S=131072 long)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing")
    ap.add_argument("--recall-rows", type=int, default=4096)
    ap.add_argument("--long", action="store_true", help="S=131072, H=32, g=16 instead")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: recall@top_k against the dense indexer and time per call "
                         "over g in {1,2,4,8,16,32} and candidate_ratio in {1,1.5,2,4} on the S=65536 workload "
                         "(top_k 2048 and 1024)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain float32 copy kernel (1 GiB read, 1 GiB written) so that "
                         "a counter run can scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the indexer runs on a single MI355X; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as syn
    import top_token_selection_amd as pv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {n * 4} bytes read, {n * 4} bytes written")
        del src, dst
    if args.sweep:
        sweep(args, dev, torch, np, syn, pv)
        return
    S, H, g = (131072, 32, 16) if args.long else (65536, 64, 8)
    D, top_k, ratio = 128, 2048, 2.0
    K = pv.candidate_count(top_k, ratio)
    seed = 1004 if args.long else 1003
    log(f"drawing prefill S={S} H={H} D={D} on the device")
    cfg = syn.long_prefill_device(dev, S=S, H=H, g=g, seed=seed)
    q, k = cfg["q"], cfg["k"]
    torch.cuda.synchronize()

    ws_bytes = max(pv.prefill_workspace_bytes(S, H, D, top_k, g, ratio, m, torch.bfloat16)
                   for m in ("refine", "reuse"))
    log(f"workspace {ws_bytes / 2**30:.1f} GiB, output {S * H * top_k * 4 / 2**30:.1f} GiB")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((S, H, top_k), dtype=torch.int32, device=dev)

    def refine():
        pv.index_prefill(q, k, top_k, g, ratio, "refine", workspace=ws, out=out)

    rng = np.random.default_rng(7)
    ri = rng.integers(g, S, max(args.recall_rows, 1))
    rh = rng.integers(0, H, max(args.recall_rows, 1)).astype(np.int32)
    ri_d = torch.from_numpy(ri).to(dev)
    rh_d = torch.from_numpy(rh.astype(np.int64)).to(dev)

    log("timing Refine")
    ms, wall_ms, stages, launches = time_calls(refine, args.steps, args.warmup, pv)
    qps = S * H / (ms / 1e3)
    log(f"Refine {ms:.2f} ms/step ({qps:.3e} queries/s); stages {stages}")
    ref_rows = out[ri_d, rh_d].cpu().numpy()

    reuse_ms = reuse_stages = None
    if not args.no_reuse:
        def reuse():
            pv.index_prefill(q, k, top_k, g, ratio, "reuse", workspace=ws, out=out)
        log("timing Reuse")
        reuse_ms, _, reuse_stages, _ = time_calls(reuse, args.steps, args.warmup, pv)
        log(f"Reuse {reuse_ms:.2f} ms/step")

    # ---------------------------------------- dense indexer (comparison)
    dense_ms = dense_stages = None
    if not args.no_dense:
        def dense():
            pv.dense_index(q, k, top_k, workspace=ws, out=out)
        log("timing the dense indexer")
        dense_ms, _, dense_stages, _ = time_calls(dense, max(1, args.steps // 2), 1, pv)
        log(f"dense {dense_ms:.2f} ms/step")

    # ------------------------------------------------------------ roofline
    sum_n, sum_nk = prefix_sums(S, g, K)
    scan_flops = 2.0 * D * H * sum_n
    gather_bytes = float(H * D * 2 * sum_nk)
    out_bytes = float(S * H * top_k * 4)
    work = {
        # algorithmic work per launch of each kernel stage
        "scan": ("mfma", scan_flops, "TFLOP/s", BF16_PEAK),
        "refine": ("hbm", gather_bytes + out_bytes + S * H * D * 2 + H * sum_nk * 4, "GB/s", HBM_PEAK),
    }
    dom = max(stages, key=lambda s: stages[s])
    roof = None
    if dom in work:
        bound, amount, unit, peak = work[dom]
        t = stages[dom] / 1e3 / max(1, launches.get(dom, 1))
        achieved = amount / max(1, launches.get(dom, 1)) / t
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        traffic = counted_traffic(dom, S, H, g)
        roof = {"bound": bound, "kernel": dom, "achieved": achieved / scale, "peak": peak / scale,
                "unit": unit, "frac": achieved / peak, "traffic": traffic,
                "achieved_basis": "algorithmic work per launch / launch time"}
        if traffic is not None and bound == "hbm":
            # the bytes the counters saw leave or reach the L2 (a part of the
            # gathered rows hits in L2): the HBM-side rate beside the
            # algorithmic one
            roof["traffic_GBps"] = traffic / t / 1e9
            roof["traffic_frac"] = traffic / t / peak
    scan_t = stages.get("scan", 0.0) / 1e3
    scan_roof = {"bound": "mfma", "achieved": scan_flops / scan_t / 1e12 if scan_t else None,
                 "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
                 "frac": scan_flops / scan_t / BF16_PEAK if scan_t else None}

    # ---------------------------------------------------------------- recall
    recall = None
    qh = kh = None
    if args.recall_rows > 0 or not args.no_cpu_baseline:
        log("copying inputs to the host for the oracle")
        qh = syn.bf16_tensor_to_bits(q)
        kh = syn.bf16_tensor_to_bits(k)
    if args.recall_rows > 0:
        from oracle.pool import OraclePool
        # the dense oracle's rows, and the group-prefix dense rows (the
        # query's own top_k over its group's prefix [0, n_j), which leaves
        # out the keys of [g_start, i): the oracle's Refine with a candidate
        # set covering every prefix), in single-threaded processes over the
        # host's cores
        t0 = time.perf_counter()
        with OraclePool(need_bytes=qh.nbytes + kh.nbytes) as pool:
            log(f"dense and group-prefix dense oracle on {args.recall_rows} sampled rows "
                f"({pool.workers} processes)")
            qr, kr = pool.put(qh), pool.put(kh)
            chunks = [c for c in np.array_split(np.arange(len(ri)), 4 * pool.workers) if len(c)]
            tasks = [("dense_rows", dict(q=qr, k=kr, rows_i=ri[c], rows_h=rh[c], top_k=top_k)) for c in chunks]
            tasks += [("prefill_rows", dict(q=qr, k=kr, rows_i=ri[c], rows_h=rh[c], top_k=top_k, g=g,
                                            candidate_ratio=S / top_k, mode="refine")) for c in chunks]
            res = pool.map(tasks)
        dense_rows = np.concatenate([r[0] for r in res[:len(chunks)]])
        gp_rows = np.concatenate([r[0] for r in res[len(chunks):]])
        dense_s = time.perf_counter() - t0
        pv.index_prefill(q, k, top_k, g, ratio, "reuse", workspace=ws, out=out)
        reu_rows = out[ri_d, rh_d].cpu().numpy()

        def rec(rows, ref):
            vals = []
            for a, b in zip(rows, ref):
                bs = set(b[b >= 0].tolist())
                vals.append(len(set(a[a >= 0].tolist()) & bs) / len(bs))
            return float(np.mean(vals))
        recall = {"refine": rec(ref_rows, dense_rows), "reuse": rec(reu_rows, dense_rows),
                  "rows": int(args.recall_rows),
                  "sample": "positions uniform in [g, S), heads uniform, seed 7", "oracle_s": dense_s,
                  "vs_group_prefix_dense": {"refine": rec(ref_rows, gp_rows), "reuse": rec(reu_rows, gp_rows)}}
        log(f"recall@{top_k}: {recall}")

    # ------------------------------------ downstream sparse attention
    attention = None
    if not args.no_attention:
        log("drawing values (Pareto-norm, like the keys) for the sparse attention")
        v = syn.pareto_keys_device(S, H, D, seed + 2000, dev)
        aout = torch.empty((S, H, D), dtype=torch.float32, device=dev)
        attention = {}
        for mode in ("refine", "reuse"):
            pv.index_prefill(q, k, top_k, g, ratio, mode, workspace=ws, out=out)
            # Reuse rows are shared by the members of a group: the grouped
            # attention gathers each group's rows once
            gg = g if mode == "reuse" else None
            ams, _, _, _ = time_calls(lambda: pv.sparse_attention(q, k, v, out, out=aout, g=gg),
                                      max(1, args.steps // 2), 1, pv)
            # algorithmic bytes: every valid entry's key and value row, plus
            # the query, index row and output row of every (position, head)
            nvalid = float((out >= 0).sum().item())
            # algorithmic bytes: the key and value rows of every valid entry
            # (of every group's row when rows are shared), the queries, the
            # index rows read and the output
            nrows_read = S * H if gg is None else ((S + g - 1) // g) * H
            ngath = nvalid if gg is None else nvalid / g
            abytes = ngath * D * 2 * 2 + S * H * (D * 2 + D * 4) + nrows_read * top_k * 4
            attention[mode] = {"ms": ams, "queries_per_s": S * H / (ams / 1e3), "valid_entries": nvalid,
                               "grouped": gg is not None, "gathered_bytes": ngath * D * 2 * 2,
                               "algorithmic_GBps": abytes / (ams / 1e3) / 1e9}
            log(f"sparse attention on {mode} rows: {ams:.2f} ms ({abytes / (ams / 1e3) / 1e9:.0f} GB/s of row reads)")
        del v, aout
        torch.cuda.empty_cache()

    # ------------------------------- literal per-position Refine (comparison)
    literal = None
    if not args.no_literal:
        Hl = 8
        ql = q[:, :Hl].contiguous()
        kl = k[:, :Hl].contiguous()
        lout = torch.empty((S, Hl, top_k), dtype=torch.int32, device=dev)
        lws = torch.empty(pv.prefill_workspace_bytes(S, Hl, D, top_k, g, ratio, "refine_literal", torch.bfloat16),
                          dtype=torch.uint8, device=dev)

        def lit():
            pv.index_prefill(ql, kl, top_k, g, ratio, "refine_literal", workspace=lws, out=lout)
        log(f"timing the literal per-position Refine on {Hl} heads")
        lms, _, lst, _ = time_calls(lit, max(1, args.steps // 2), 1, pv)
        literal = {"heads": Hl, "ms_per_step": lms, "queries_per_s": S * Hl / (lms / 1e3), "stage_ms": lst}
        # recall@top_k on 512 rows of these heads against the dense indexer (GPU)
        if args.recall_rows > 0:
            lrng = np.random.default_rng(9)
            li = torch.from_numpy(lrng.integers(g, S, 512)).to(dev)
            lh = torch.from_numpy(lrng.integers(0, Hl, 512)).to(dev)
            lit_rows = lout[li, lh].cpu().numpy()
            pv.index_prefill(ql, kl, top_k, g, ratio, "refine", workspace=lws, out=lout)
            one_rows = lout[li, lh].cpu().numpy()
            del lws
            pv.dense_index(ql, kl, top_k, out=lout, max_workspace_bytes=48 << 30)
            den_rows = lout[li, lh].cpu().numpy()

            def rec3(a_rows):
                return float(np.mean([len(set(a[a >= 0].tolist()) & set(b[b >= 0].tolist()))
                                      / max(1, int((b >= 0).sum())) for a, b in zip(a_rows, den_rows)]))
            literal["recall"] = {"literal": rec3(lit_rows), "refine": rec3(one_rows), "rows": 512,
                                 "against": "dense indexer (GPU)",
                                 "sample": f"positions uniform in [g, S), heads uniform in [0, {Hl}), seed 9"}
        log(f"literal per-position Refine: {lms:.2f} ms/step on {Hl} heads; {literal.get('recall')}")
        del ql, kl, lout
        torch.cuda.empty_cache()

    # ---------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from oracle.pool import OraclePool, workers_default
        rng = np.random.default_rng(11)
        G = (S + g - 1) // g
        done_rows = 0
        t0 = time.perf_counter()
        ngroups = 0
        log(f"timing the oracle on one core for about {args.cpu_seconds:.0f} s")
        while time.perf_counter() - t0 < args.cpu_seconds:
            hh = rng.integers(0, H, 1).astype(np.int32)
            jj = rng.integers(0, G, 1)
            oracle.prefill_groups(qh, kh, hh, jj, top_k, g, ratio, "refine")
            done_rows += int(min(g, S - jj[0] * g))
            ngroups += 1
        el = time.perf_counter() - t0
        single = {"value": done_rows / el, "unit": "queries/s", "cores": 1, "groups": ngroups, "seconds": el}
        log(f"oracle, one core: {single['value']:.2f} queries/s")
        nw = workers_default()
        log(f"timing the oracle on {nw} cores (one single-threaded process each) for about {args.cpu_seconds:.0f} s")
        with OraclePool(workers=nw, need_bytes=qh.nbytes + kh.nbytes) as pool:
            qr, kr = pool.put(qh), pool.put(kh)
            w0 = time.perf_counter()
            res = pool.map([("timed_groups", dict(q=qr, k=kr, seconds=args.cpu_seconds, seed=11 + 1000 * (w + 1),
                                                  top_k=top_k, g=g, candidate_ratio=ratio, mode="refine"))
                            for w in range(nw)])
            wall = time.perf_counter() - w0
        rows_all = sum(r[0] for r in res)
        rate = sum(r[0] / r[2] for r in res)
        cpu = {"value": rate, "unit": "queries/s", "cores": nw, "kind": "oracle",
               "sample": f"PIVOT-Refine groups (all {g} members each) drawn uniformly over (head, group) of this "
                         f"workload: {nw} single-threaded C oracle processes for {args.cpu_seconds:.0f} s each "
                         f"({sum(r[1] for r in res)} groups), value = sum of the per-process rates; "
                         f"one core alone: {single['value']:.1f} queries/s ({ngroups} groups, seed 11)",
               "single_core": single,
               "all_core_wall": {"rows": rows_all, "seconds": wall, "queries_per_s": rows_all / wall},
               "cpu_model": cpu_model(), "nproc": os.cpu_count()}
        log(f"oracle, {nw} cores: {rate:.2f} queries/s")
    del ws, out, q, k, cfg
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        decode = {}
        for gd in (2, 4):
            log(f"drawing decode g={gd}")
            dc = syn.decode_step_device(dev, g=gd)
            ctx = dc["ctx_lens"]
            nbytes = float(ctx.sum()) * 8 * D * 2
            dws = torch.empty(max(pv.decode_workspace_bytes(ctx, gd, 8, D, top_k, ratio, m, torch.bfloat16)
                                  for m in ("refine", "reuse")), dtype=torch.uint8, device=dev)
            dout = torch.empty((len(ctx) * gd, 8, top_k), dtype=torch.int32, device=dev)
            for mode in ("refine", "reuse"):
                def step():
                    pv.index_decode(dc["q"], dc["k_cache"], ctx, gd, top_k, ratio, mode, workspace=dws, out=dout)
                dms, _, dst, _ = time_calls(step, args.steps * 4, args.warmup, pv)
                t_scan = dst.get("decode_scan", 0.0) / 1e3
                decode[f"g{gd}_{mode}"] = {
                    "us_per_step": dms * 1e3, "stage_ms": dst,
                    "scan_GBps": nbytes / t_scan / 1e9 if t_scan else None,
                    "scan_hbm_frac": nbytes / t_scan / HBM_PEAK if t_scan else None,
                    "key_bytes": nbytes}
                log(f"decode g={gd} {mode}: {dms * 1e3:.0f} us/step, scan {nbytes / t_scan / 1e9:.0f} GB/s")
            del dc, dws, dout
            torch.cuda.empty_cache()

    # ----------------------------------------------------- other workloads
    configs = None
    if not args.no_configs:
        configs = {}

        def host(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        def prefill_config(name, qd, kd, tk, gg, modes, dense_too, ksteps, all_rows_recall=False):
            Sx, Hx, Dx = qd.shape
            Kx = pv.candidate_count(tk, 2.0)
            wsx = torch.empty(max(pv.prefill_workspace_bytes(Sx, Hx, Dx, tk, gg, 2.0, m, qd.dtype)
                                  for m in ("refine", "reuse")), dtype=torch.uint8, device=dev)
            outx = torch.empty((Sx, Hx, tk), dtype=torch.int32, device=dev)
            sn, _ = prefix_sums(Sx, gg, Kx)
            res = {"S": Sx, "H": Hx, "D": Dx, "top_k": tk, "g": gg, "K": Kx, "dtype": str(qd.dtype)}
            for mode in modes:
                def call():
                    pv.index_prefill(qd, kd, tk, gg, 2.0, mode, workspace=wsx, out=outx)
                cms, _, cst, _ = time_calls(call, ksteps, args.warmup, pv)
                st = cst.get("scan", 0.0) / 1e3
                res[mode] = {"ms_per_step": cms, "queries_per_s": Sx * Hx / (cms / 1e3), "stage_ms": cst,
                             "scan_mfma_frac": 2.0 * Dx * Hx * sn / st / BF16_PEAK if st else None}
                log(f"{name} {mode}: {cms:.3f} ms/step ({Sx * Hx / (cms / 1e3):.3e} queries/s)")
            if dense_too:
                def dcall():
                    pv.dense_index(qd, kd, tk, workspace=wsx, out=outx)
                cms, _, cst, _ = time_calls(dcall, ksteps, args.warmup, pv)
                res["dense"] = {"ms_per_step": cms, "queries_per_s": Sx * Hx / (cms / 1e3), "stage_ms": cst}
                log(f"{name} dense: {cms:.3f} ms/step")
            if all_rows_recall:
                # recall@top_k of every row (positions >= 1) against the dense
                # indexer (the GPU's: bit-exact to the oracle on integer
                # inputs, tie-tolerant on Gaussian ones)
                dref = pv.dense_index(qd, kd, tk, max_workspace_bytes=48 << 30).view(Sx * Hx, tk)
                rec = {}
                for mode in modes:
                    rows = pv.index_prefill(qd, kd, tk, gg, 2.0, mode, workspace=wsx).view(Sx * Hx, tk)
                    rec[mode] = recall_rows(rows, dref, skip_first_rows=1, H=Hx)
                rec.update({"rows": (Sx - 1) * Hx, "against": "dense indexer (GPU), every row with i >= 1"})
                res["recall"] = rec
                log(f"{name} recall@{tk}: {rec}")
                del dref
            del wsx, outx
            return res

        tc = syn.tiny_prefill()
        configs["tiny"] = prefill_config("tiny S=1024 H=8 D=64 fp32", host(tc["q"]), host(tc["k"]), 64, 8,
                                         ("refine", "reuse"), True, args.steps * 4, all_rows_recall=True)
        ic = syn.int_prefill()
        configs["int16k"] = prefill_config("S=16384 H=16 integer bf16", host(ic["q"]), host(ic["k"]), 512, 8,
                                           ("refine", "reuse"), False, args.steps * 2, all_rows_recall=True)
        del tc, ic
        log("drawing the long prefill S=131072 H=32 g=16 on the device")
        lc = syn.long_prefill_device(dev, S=131072, H=32, g=16, seed=1004)
        lres = prefill_config("long S=131072 H=32 g=16", lc["q"], lc["k"], 2048, 16, ("refine", "reuse"),
                              False, max(2, args.steps // 2))
        # recall@2048 on a 4096-row sample against the dense oracle and the
        # group-prefix dense oracle rows (single-threaded processes over the
        # host's cores)
        if args.recall_rows > 0:
            from oracle.pool import OraclePool
            Sl, Hl, gl = 131072, 32, 16
            rng = np.random.default_rng(13)
            li_h = rng.integers(16, Sl, 4096)
            lh_h = rng.integers(0, Hl, 4096).astype(np.int32)
            li, lh = torch.from_numpy(li_h).to(dev), torch.from_numpy(lh_h.astype(np.int64)).to(dev)
            lws = torch.empty(pv.prefill_workspace_bytes(Sl, Hl, 128, 2048, gl, 2.0, "refine", torch.bfloat16),
                              dtype=torch.uint8, device=dev)
            lout = torch.empty((Sl, Hl, 2048), dtype=torch.int32, device=dev)
            rows = {}
            for mode in ("refine", "reuse"):
                pv.index_prefill(lc["q"], lc["k"], 2048, gl, 2.0, mode, workspace=lws, out=lout)
                rows[mode] = lout[li, lh].cpu().numpy()
            del lws, lout
            lqh, lkh = syn.bf16_tensor_to_bits(lc["q"]), syn.bf16_tensor_to_bits(lc["k"])
            t0 = time.perf_counter()
            with OraclePool(need_bytes=lqh.nbytes + lkh.nbytes) as pool:
                qr, kr = pool.put(lqh), pool.put(lkh)
                chunks = [c for c in np.array_split(np.arange(4096), 4 * pool.workers) if len(c)]
                tasks = [("dense_rows", dict(q=qr, k=kr, rows_i=li_h[c], rows_h=lh_h[c], top_k=2048))
                         for c in chunks]
                tasks += [("prefill_rows", dict(q=qr, k=kr, rows_i=li_h[c], rows_h=lh_h[c], top_k=2048, g=gl,
                                                candidate_ratio=Sl / 2048, mode="refine")) for c in chunks]
                res = pool.map(tasks)
            del lqh, lkh
            drows = np.concatenate([r[0] for r in res[:len(chunks)]])
            gprows = np.concatenate([r[0] for r in res[len(chunks):]])

            def rec2(a_rows, ref):
                vals = []
                for a, b in zip(a_rows, ref):
                    bs = set(b[b >= 0].tolist())
                    vals.append(len(set(a[a >= 0].tolist()) & bs) / len(bs))
                return float(np.mean(vals))
            lres["recall"] = {"refine": rec2(rows["refine"], drows), "reuse": rec2(rows["reuse"], drows),
                              "rows": 4096, "against": "dense oracle",
                              "sample": "positions uniform in [16, S), heads uniform, seed 13",
                              "oracle_s": time.perf_counter() - t0,
                              "vs_group_prefix_dense": {"refine": rec2(rows["refine"], gprows),
                                                        "reuse": rec2(rows["reuse"], gprows)}}
            log(f"long recall@2048: {lres['recall']}")
        configs["long131k"] = lres
        del lc
        torch.cuda.empty_cache()

    line = {
        "metric": "indexed queries/s (Refine, S=64K prefill) + decode us/step; % MFMA/HBM roofline",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (device-drawn AR(1) queries, Pareto-norm keys; seeds in synthetic/)",
        "config": {"workload": f"PIVOT-Refine prefill S={S} H={H} D={D} bf16 top_k={top_k} g={g} K={K}",
                   "mode": "refine", "S": S, "H": H, "D": D, "top_k": top_k, "g": g, "K": K},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": {
            "wall_ms_per_step": wall_ms,
            "stage_ms": stages,
            "stage_launches": launches,
            "scan_roofline": scan_roof,
            "scan_flops": scan_flops,
            "refine_gather_bytes": gather_bytes,
            "output_bytes": out_bytes,
            "reuse_ms_per_step": reuse_ms,
            "reuse_queries_per_s": S * H / (reuse_ms / 1e3) if reuse_ms else None,
            "reuse_stage_ms": reuse_stages,
            "dense_ms_per_step": dense_ms,
            "dense_queries_per_s": S * H / (dense_ms / 1e3) if dense_ms else None,
            "dense_stage_ms": dense_stages,
            "indexer_speedup_vs_dense": ({"refine": dense_ms / ms, "reuse": dense_ms / reuse_ms if reuse_ms else None}
                                         if dense_ms else None),
            "decode": decode,
            "recall": recall,
            "literal_refine": literal,
            "sparse_attention": attention,
            "configs": configs,
            "host": {"cpu": cpu_model(), "nproc": os.cpu_count(),
                     "gpu": torch.cuda.get_device_name(dev)},
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
