"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer-valued inputs (every float32 score exact) are compared bit for bit:
indices, order, -1 padding and scores. Gaussian inputs are compared
tie-tolerantly (tests/parity.py). Sizes span several scan tiles (256 groups)
and ragged tails; the degenerate cases (all-equal scores, one-key prefixes,
top_k beyond the prefix) are included.
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


def dev_tensor(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


@pytest.fixture(scope="module")
def pv():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import top_token_selection_amd as pv
    return pv


def run_prefill(pv, q, k, top_k, g, ratio, mode):
    idx, sc = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio,
                               mode=mode, return_scores=True)
    torch.cuda.synchronize()
    return parity.to_host(idx), parity.to_host(sc)


def prefill_limits(S, g):
    i = np.arange(S)
    return np.maximum((i // g) * g, 1)[:, None]


# ----------------------------------------------------------- bit-exact

EXACT_CASES = [
    # S, H, D, top_k, g, ratio, dtype
    (1024, 8, 64, 64, 8, 2.0, "f32"),     # the tiny workload's integer twin
    (700, 3, 128, 16, 8, 2.0, "bf16"),    # ragged tail, several tiles of rows
    (600, 2, 64, 24, 3, 1.5, "bf16"),     # non-power-of-two groups
    (513, 2, 128, 8, 1, 2.0, "bf16"),     # g = 1
    (300, 2, 64, 40, 16, 2.0, "f32"),     # top_k beyond early prefixes
    (2100, 1, 128, 100, 8, 2.0, "bf16"),  # > 8 scan tiles, rows that need sampling
    (1500, 3, 128, 37, 8, 2.0, "bf16"),   # odd top_k: output rows off 16-byte alignment
    (900, 2, 64, 101, 4, 1.5, "f32"),     # odd top_k and K = floor(151.5)
    (800, 2, 128, 50, 8, 1.0, "bf16"),    # ratio 1: K = top_k
    (1200, 2, 128, 30, 8, 4.0, "bf16"),   # ratio 4: K = 4 top_k
    (2000, 2, 64, 48, 32, 2.0, "bf16"),   # g = 32: four blocks of 8 members per group
]


@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("S,H,D,top_k,g,ratio,dtype", EXACT_CASES)
def test_prefill_bit_exact_integer_inputs(pv, mode, S, H, D, top_k, g, ratio, dtype):
    print(f"\n[prefill exact] S={S} H={H} D={D} k={top_k} g={g} r={ratio} {dtype} {mode}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), 7000 + S + g, a, dtype)
    k = syn.integers((S, H, D), 8000 + S + g, a, dtype)
    gi, gs = run_prefill(pv, q, k, top_k, g, ratio, mode)
    oi, os_ = oracle.prefill(q, k, top_k, g, ratio, mode)
    np.testing.assert_array_equal(gi, oi)
    if dtype == "bf16" or S % g == 0 and (g & (g - 1)) == 0:
        # every proxy is exact (power-of-two group of small integers, or a
        # bf16 proxy whose products and sums stay within float32's 24 bits)
        np.testing.assert_array_equal(gs, os_)
    else:
        # fp32 proxy of a ragged group (sum / m, m not a power of two) is
        # rounded once; float32 accumulation order then moves scores by ulps
        np.testing.assert_allclose(gs, os_, rtol=4 * 2.0 ** -23, atol=0)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("S,H,D,top_k,g,ratio,dtype", EXACT_CASES)
def test_index_only_bit_exact(pv, mode, S, H, D, top_k, g, ratio, dtype):
    """Indices without scores take the wavefront bucket sorts (Refine: per
    query; Reuse: per group, one wavefront per row of survivors); they must
    equal the oracle's rows exactly as well."""
    print(f"\n[{mode} index-only] S={S} H={H} D={D} k={top_k} g={g} r={ratio} {dtype}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), 7000 + S + g, a, dtype)
    k = syn.integers((S, H, D), 8000 + S + g, a, dtype)
    idx = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio,
                           mode=mode)
    torch.cuda.synchronize()
    oi, _ = oracle.prefill(q, k, top_k, g, ratio, mode)
    np.testing.assert_array_equal(parity.to_host(idx), oi)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_index_only_gaussian_large_top_k(pv, mode):
    """Gaussian inputs with top_k = 2048 (the largest top_k the wavefront
    sorts take) and with top_k = 2500 (past it: the general selectors; K =
    4000 for Refine); index-only rows equal the rows of the scored launch
    (general selectors) exactly."""
    S, H, D, g = 9000, 2, 128, 8
    q = syn.gaussian((S, H, D), 7301, "bf16")
    k = syn.gaussian((S, H, D), 7302, "bf16")
    for top_k, ratio in ((2048, 2.0), (2500, 1.6)):
        print(f"\n[{mode} index-only gaussian] S={S} H={H} k={top_k} r={ratio}", flush=True)
        qd, kd = dev_tensor(q), dev_tensor(k)
        a = pv.index_prefill(qd, kd, top_k=top_k, g=g, candidate_ratio=ratio, mode=mode)
        b, _ = pv.index_prefill(qd, kd, top_k=top_k, g=g, candidate_ratio=ratio, mode=mode,
                                return_scores=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(parity.to_host(a), parity.to_host(b))


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_heavy_ties_at_the_boundary(pv, mode):
    """0/1 queries and keys: scores take ~25 values over 4096 candidates, so
    hundreds of keys tie at the selection boundary (the per-query bucket of
    the boundary overflows its staging and the exact general path takes
    over, index-only and with scores)."""
    print(f"\n[heavy ties] {mode}", flush=True)
    S, H, D, top_k, g = 4104, 1, 64, 2048, 8
    rng = np.random.default_rng(77)
    q = syn.to_bf16_bits(rng.integers(0, 2, (S, H, D)).astype(np.float32))
    k = syn.to_bf16_bits(rng.integers(0, 2, (S, H, D)).astype(np.float32))
    oi, os_ = oracle.prefill(q, k, top_k, g, 2.0, mode)
    gi, gs = run_prefill(pv, q, k, top_k, g, 2.0, mode)
    np.testing.assert_array_equal(gi, oi)
    np.testing.assert_array_equal(gs, os_)
    only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, mode=mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(only), oi)


def test_refine_large_tie_group_among_staged_keys(pv):
    """One key vector repeated at every 13th position scores far above the
    others for every query (queries in [0, 3], the repeated key all 3s,
    the rest in [-3, 3]), so each query's best fine bucket holds every copy
    in its prefix: fewer than 256 copies in early rows (the staged-slot
    scatter with one long bucket), up to 315 in late ones (past the 8-bit
    slots: the exact general path). K = 2048, top_k = 1024; bit-exact."""
    print("\n[large tie group] refine", flush=True)
    S, H, D, top_k, g = 4104, 1, 64, 1024, 8
    rng = np.random.default_rng(4242)
    q = rng.integers(0, 4, (S, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, (S, H, D)).astype(np.float32)
    hot = np.arange(5, S, 13)
    k[hot] = 3.0
    q, k = syn.to_bf16_bits(q), syn.to_bf16_bits(k)
    oi, os_ = oracle.prefill(q, k, top_k, g, 2.0, "refine")
    # the design holds: late rows start with every copy in the prefix
    last = oi[S - 1, 0]
    n_hot = int(np.sum(hot < (S - 1) // g * g))
    assert n_hot >= 256 and np.array_equal(last[:n_hot], hot[:n_hot])
    gi, gs = run_prefill(pv, q, k, top_k, g, 2.0, "refine")
    np.testing.assert_array_equal(gi, oi)
    np.testing.assert_array_equal(gs, os_)
    only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, mode="refine")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(only), oi)


@pytest.mark.parametrize("S,H,D,top_k,dtype", [(1024, 8, 64, 64, "f32"), (700, 3, 128, 32, "bf16")])
def test_dense_bit_exact_integer_inputs(pv, S, H, D, top_k, dtype):
    print(f"\n[dense exact] S={S} H={H} D={D} k={top_k} {dtype}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), 7100 + S, a, dtype)
    k = syn.integers((S, H, D), 8100 + S, a, dtype)
    idx, sc = pv.dense_index(dev_tensor(q), dev_tensor(k), top_k=top_k, return_scores=True)
    only = pv.dense_index(dev_tensor(q), dev_tensor(k), top_k=top_k)
    torch.cuda.synchronize()
    oi, os_ = oracle.dense(q, k, top_k)
    np.testing.assert_array_equal(parity.to_host(idx), oi)
    np.testing.assert_array_equal(parity.to_host(sc), os_)
    np.testing.assert_array_equal(parity.to_host(only), oi)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("g", [2, 4])
def test_decode_bit_exact_integer_inputs(pv, mode, g):
    print(f"\n[decode exact] g={g} {mode}", flush=True)
    H, D, top_k = 4, 128, 32
    ctx = np.array([1, 5, 64, 300, 1000, 77], np.int64)
    kc = syn.integers((int(ctx.sum()), H, D), 9001, 4, "bf16")
    q = syn.integers((len(ctx) * g, H, D), 9002 + g, 4, "bf16")
    idx, sc = pv.index_decode(dev_tensor(q), dev_tensor(kc), ctx, g, top_k=top_k, mode=mode, return_scores=True)
    only = pv.index_decode(dev_tensor(q), dev_tensor(kc), ctx, g, top_k=top_k, mode=mode)
    torch.cuda.synchronize()
    oi, os_ = oracle.decode(q, kc, ctx, g, top_k, 2.0, mode)
    np.testing.assert_array_equal(parity.to_host(idx), oi)
    np.testing.assert_array_equal(parity.to_host(sc), os_)
    np.testing.assert_array_equal(parity.to_host(only), oi)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_decode_long_rows_bit_exact(pv, mode):
    """Contexts spanning several 4096-key filter chunks with ragged tails
    and one of a single key, top_k=2048 (K=4096), integer-valued inputs.
    The queries of one sequence are zero: every key of its rows ties, the
    rows overflow the survivor buffers and take the exact fallback. Scored
    and index-only launches (the latter takes the wavefront select for
    Reuse) both equal the oracle."""
    H, D, top_k, g = 2, 128, 2048, 2
    ctx = np.array([4096, 70001, 1, 12289, 33000, 130000, 2500], np.int64)
    print(f"\n[decode long exact] {mode} ctx={ctx.tolist()}", flush=True)
    kc = syn.integers((int(ctx.sum()), H, D), 9101, 4, "bf16")
    q = syn.integers((len(ctx) * g, H, D), 9102, 4, "bf16")
    q[3 * g:4 * g] = 0
    qd, kd = dev_tensor(q), dev_tensor(kc)
    idx, sc = pv.index_decode(qd, kd, ctx, g, top_k=top_k, mode=mode, return_scores=True)
    only = pv.index_decode(qd, kd, ctx, g, top_k=top_k, mode=mode)
    torch.cuda.synchronize()
    oi, os_ = oracle.decode(q, kc, ctx, g, top_k, 2.0, mode)
    np.testing.assert_array_equal(parity.to_host(idx), oi)
    np.testing.assert_array_equal(parity.to_host(sc), os_)
    np.testing.assert_array_equal(parity.to_host(only), oi)


# ------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_all_scores_equal_ties_by_index(pv, mode):
    """Zero queries: every score is 0, so every row is the smallest indices
    (exercises the tie resolution and the exact fallback)."""
    print(f"\n[ties] {mode}", flush=True)
    S, H, D, top_k, g = 900, 2, 64, 20, 4
    q = np.zeros((S, H, D), np.float32)
    k = syn.integers((S, H, D), 31, 3, "f32")
    gi, gs = run_prefill(pv, q, k, top_k, g, 2.0, mode)
    oi, os_ = oracle.prefill(q, k, top_k, g, 2.0, mode)
    np.testing.assert_array_equal(gi, oi)
    np.testing.assert_array_equal(gs, os_)
    only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, mode=mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(only), oi)


def test_tiny_and_degenerate_shapes(pv):
    for (S, H, D, top_k, g) in [(1, 1, 64, 4, 8), (5, 2, 64, 3, 8), (9, 1, 128, 16, 4), (64, 1, 64, 64, 64)]:
        for mode in ("refine", "reuse"):
            print(f"\n[shape] S={S} H={H} D={D} k={top_k} g={g} {mode}", flush=True)
            q = syn.integers((S, H, D), 41 + S, 4, "bf16")
            k = syn.integers((S, H, D), 42 + S, 4, "bf16")
            gi, gs = run_prefill(pv, q, k, top_k, g, 2.0, mode)
            oi, os_ = oracle.prefill(q, k, top_k, g, 2.0, mode)
            np.testing.assert_array_equal(gi, oi)
            np.testing.assert_array_equal(gs, os_)
            only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, mode=mode)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(parity.to_host(only), oi)


def test_refine_with_K_covering_prefix_equals_group_prefix_dense(pv):
    S, H, D, top_k, g = 256, 2, 64, 8, 8
    q = syn.integers((S, H, D), 51, 4, "bf16")
    k = syn.integers((S, H, D), 52, 4, "bf16")
    ratio = 512 / top_k  # K = 512 >= S
    gi, _ = run_prefill(pv, q, k, top_k, g, ratio, "refine")
    oi, _ = oracle.prefill(q, k, top_k, g, ratio, "refine")
    np.testing.assert_array_equal(gi, oi)


def test_g1_reuse_equals_dense_on_gpu(pv):
    S, H, D, top_k = 400, 2, 128, 16
    q = syn.gaussian((S, H, D), 61, "bf16")
    k = syn.gaussian((S, H, D), 62, "bf16")
    a = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=1, mode="reuse")
    b = pv.dense_index(dev_tensor(q), dev_tensor(k), top_k=top_k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(a), parity.to_host(b))


def test_head_chunking_matches_single_pass(pv):
    """A workspace for one head per pass gives the same result."""
    S, H, D, top_k, g = 600, 4, 64, 16, 8
    q = syn.gaussian((S, H, D), 71, "bf16")
    k = syn.gaussian((S, H, D), 72, "bf16")
    full = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g)
    one = pv.prefill_workspace_bytes(S, 1, D, top_k, g, 2.0, "refine", torch.bfloat16)
    chunked = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, max_workspace_bytes=one)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(full), parity.to_host(chunked))


def test_deterministic_repeat(pv):
    S, H, D, top_k, g = 1500, 2, 128, 64, 8
    q = dev_tensor(syn.gaussian((S, H, D), 81, "bf16"))
    k = dev_tensor(syn.gaussian((S, H, D), 82, "bf16"))
    for mode in ("refine", "reuse"):
        a = pv.index_prefill(q, k, top_k=top_k, g=g, mode=mode, return_scores=True)
        b = pv.index_prefill(q, k, top_k=top_k, g=g, mode=mode, return_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------ tolerant (Gaussian)

@pytest.mark.parametrize("mode", ["refine", "reuse"])
def test_tiny_workload_gaussian_tolerant(pv, mode):
    """The tiny workload (S=1024, H=8, D=64, fp32 N(0,1), top_k=64, g=8)."""
    print(f"\n[tiny gaussian] {mode}", flush=True)
    cfg = syn.tiny_prefill(integer=False)
    q, k = cfg["q"], cfg["k"]
    S, H, D = q.shape
    top_k, g = cfg["top_k"], cfg["g"]
    gi, gs = run_prefill(pv, q, k, top_k, g, 2.0, mode)
    oi, os_ = oracle.prefill(q, k, top_k, g, 2.0, mode)
    K = oracle.candidate_count(top_k, 2.0)
    valid = np.minimum(top_k, np.minimum(K, prefill_limits(S, g)))
    parity.structure_ok(gi, gs, prefill_limits(S, g), valid)
    errs = []
    qv = q.astype(np.float64)
    for h in range(H):
        kv_all = parity.key_values(k, h)
        for j in range(S // g):
            n = max(j * g, 1)
            proxy = oracle.proxy(q, g, h, j).astype(np.float64)
            cand = None
            if mode == "refine":
                cand, _ = oracle.prefill_candidates(q, k, h, j, top_k, g, 2.0)
            for i in range(j * g, j * g + g):
                avec = qv[i, h] if mode == "refine" else proxy
                e = parity.row_match(gi[i, h], gs[i, h], oi[i, h], os_[i, h], avec, kv_all[:n], proxy=proxy,
                                     cand_idx=cand)
                if e:
                    errs.append((i, h, e))
    assert not errs, errs[:5]


# ------------------------------------------------- proxy rounding on the GPU

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_proxy_rounding_matches_hand_derived_values(pv, dtype):
    """The proxies of tests/test_oracle_proxy_pins.py, read back through
    Reuse scores: key c of the prefix is the unit vector e_c, so the proxy
    score of key c is the proxy's component c, exactly. Group 1 (positions
    8..15) holds the members whose float32 sums round (expected proxies 0,
    0.5, 0.75, 0.75 by hand); a ragged group 2 (positions 16..18) holds
    [5, 0, 0], whose float32 quotient is 0x3FD55555 (fp32) or 213/128 (bf16)."""
    from tests.test_oracle_proxy_pins import SUM_MEMBERS, SUM_PROXY, DIV_BITS
    S, H, D = 19, 1, 64
    qf = np.zeros((S, H, D), np.float32)
    qf[8:16, 0, :4] = SUM_MEMBERS
    qf[16, 0, 0] = 5.0
    kf = np.zeros((S, H, D), np.float32)
    for c in range(16):
        kf[c, 0, c] = 1.0
    q = qf if dtype == "f32" else syn.to_bf16_bits(qf)
    k = kf if dtype == "f32" else syn.to_bf16_bits(kf)
    gi, gs = run_prefill(pv, q, k, 16, 8, 2.0, "reuse")
    # group 1 sees keys 0..7: components 0..3 carry the sums, 4..7 are zero
    want = {c: float(SUM_PROXY[c]) for c in range(4)}
    want.update({c: 0.0 for c in range(4, 8)})
    order = sorted(want, key=lambda c: (-want[c], c))
    for i in range(8, 16):
        np.testing.assert_array_equal(gi[i, 0, :8], order)
        np.testing.assert_array_equal(gs[i, 0, :8], np.array([want[c] for c in order], np.float32))
    # group 2 sees keys 0..15: component 0 is the quotient, the rest zero
    for i in range(16, 19):
        assert gi[i, 0, 0] == 0
        if dtype == "f32":
            assert int(gs[i, 0, 0:1].view(np.uint32)[0]) == DIV_BITS
        else:
            assert float(gs[i, 0, 0]) == 213.0 / 128.0


# ------------------------------------------ top_k beyond the wavefront sorts

LARGE_TOPK = [
    # S, H, D, top_k, ratio, g, dtype: K = floor(top_k * ratio)
    (9000, 2, 128, 3000, 1.3, 8, "bf16"),   # K = 3900: selectors past the 2048-entry staging
    (9000, 1, 128, 4096, 1.0, 8, "bf16"),   # K = top_k = 4096: a wavefront's whole register list
    (9000, 2, 128, 2048, 4.0, 8, "bf16"),   # K = 8192: refine through global score rows
    (9000, 1, 128, 8192, 1.0, 8, "bf16"),   # top_k = K = 8192, the largest
    (9000, 1, 128, 5000, 1.5, 4, "bf16"),   # Reuse rows past 4096 (bucket sort straight to rows)
    (6000, 1, 64, 2100, 2.0, 4, "f32"),     # K = 4200 with fp32 keys, D = 64
]


@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("S,H,D,top_k,ratio,g,dtype", LARGE_TOPK)
def test_large_top_k_bit_exact_integer_inputs(pv, mode, S, H, D, top_k, ratio, g, dtype):
    """top_k above 2048 and K up to 8192 against the oracle, bit for bit on
    integer inputs (index-only and with scores)."""
    from oracle.pool import OraclePool
    print(f"\n[large top_k] S={S} H={H} D={D} k={top_k} r={ratio} g={g} {dtype} {mode}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), 7600 + top_k, a, dtype)
    k = syn.integers((S, H, D), 7700 + top_k, a, dtype)
    gi, gs = run_prefill(pv, q, k, top_k, g, ratio, mode)
    only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio, mode=mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(only), gi)
    with OraclePool() as pool:
        res = pool.map([("prefill", dict(q=pool.put(q[:, h:h + 1]), k=pool.put(k[:, h:h + 1]), top_k=top_k, g=g,
                                         candidate_ratio=ratio, mode=mode)) for h in range(H)])
    exact_scores = dtype == "bf16" or (g & (g - 1)) == 0
    for h, (oi, os_) in enumerate(res):
        np.testing.assert_array_equal(gi[:, h], oi[:, 0], err_msg=f"head {h}")
        if exact_scores:
            np.testing.assert_array_equal(gs[:, h], os_[:, 0], err_msg=f"head {h}")
        else:
            # a float32 proxy of 3 members is rounded once; float32
            # accumulation order then moves its scores by ulps
            np.testing.assert_allclose(gs[:, h], os_[:, 0], rtol=4 * 2.0 ** -23, atol=0)


@pytest.mark.parametrize("mode", ["refine", "reuse"])
@pytest.mark.parametrize("top_k,ratio,g", [(3000, 1.3, 2), (4096, 1.0, 4), (2048, 4.0, 2), (8192, 1.0, 4)])
def test_decode_large_top_k_bit_exact_integer_inputs(pv, mode, top_k, ratio, g):
    print(f"\n[decode large top_k] k={top_k} r={ratio} g={g} {mode}", flush=True)
    H, D = 2, 128
    ctx = np.array([9000, 3100, 12000, 4096, 1], np.int64)
    B = len(ctx)
    kc = syn.integers((int(ctx.sum()), H, D), 7800 + top_k, 4, "bf16")
    q = syn.integers((B * g, H, D), 7900 + top_k, 4, "bf16")
    for scores in (True, False):
        r = pv.index_decode(dev_tensor(q), dev_tensor(kc), ctx, g, top_k=top_k, candidate_ratio=ratio, mode=mode,
                            return_scores=scores)
        torch.cuda.synchronize()
        oi, os_ = oracle.decode(q, kc, ctx, g, top_k, ratio, mode)
        if scores:
            np.testing.assert_array_equal(parity.to_host(r[0]), oi)
            np.testing.assert_array_equal(parity.to_host(r[1]), os_)
        else:
            np.testing.assert_array_equal(parity.to_host(r), oi)


# ------------------------------- literal per-position Refine (comparison)

@pytest.mark.parametrize("S,H,D,top_k,g,ratio,dtype", [
    (1024, 8, 64, 64, 8, 2.0, "f32"),
    (700, 3, 128, 16, 8, 2.0, "bf16"),
    (600, 2, 64, 24, 3, 1.5, "bf16"),
    (2100, 1, 128, 100, 8, 2.0, "bf16"),
    (4500, 1, 128, 2048, 8, 4.0, "bf16"),   # K = 8192: global score rows
])
def test_literal_refine_bit_exact_integer_inputs(pv, S, H, D, top_k, g, ratio, dtype):
    """The per-position rescan (one scan row per position, the group's proxy)
    against the oracle's literal mode, with scores and index-only."""
    print(f"\n[literal exact] S={S} H={H} D={D} k={top_k} g={g} r={ratio} {dtype}", flush=True)
    a = 8 if dtype == "f32" else 4
    q = syn.integers((S, H, D), 7400 + S + g, a, dtype)
    k = syn.integers((S, H, D), 8400 + S + g, a, dtype)
    gi, gs = run_prefill(pv, q, k, top_k, g, ratio, "refine_literal")
    oi, os_ = oracle.prefill(q, k, top_k, g, ratio, "refine_literal")
    np.testing.assert_array_equal(gi, oi)
    if dtype == "bf16" or (S % g == 0 and (g & (g - 1)) == 0):
        np.testing.assert_array_equal(gs, os_)
    else:
        np.testing.assert_allclose(gs, os_, rtol=4 * 2.0 ** -23, atol=0)
    only = pv.index_prefill(dev_tensor(q), dev_tensor(k), top_k=top_k, g=g, candidate_ratio=ratio,
                            mode="refine_literal")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(parity.to_host(only), oi)
