"""PIVOT query-group indexer on MI355X -- Python binding of ``libpivot.so``.

Argument marshalling only: every step of the indexer runs in the HIP
kernels of ``libpivot.so`` (C ABI in ``include/pivot.h``). PyTorch provides
device memory and the current stream. There is no other implementation to
fall back to: importing this package without the built library raises.

    idx = index_prefill(q, k, top_k=64, g=8, candidate_ratio=2.0, mode="refine")
    idx = index_decode(q, k_cache, ctx_lens, g=2, top_k=2048)
    idx = dense_index(q, k, top_k=64)

q, k: (S, H, D) contiguous device tensors, float32 or bfloat16. Results are
int32 (rows, H, top_k) tensors with -1 padding (and float32 scores with -inf
padding when ``return_scores=True``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpivot.so")

PIVOT_OK, PIVOT_EINVAL, PIVOT_EUNSUPPORTED, PIVOT_EWORKSPACE, PIVOT_EHIP = 0, -1, -2, -3, -4
PIVOT_F32, PIVOT_BF16 = 0, 1
PIVOT_REFINE, PIVOT_REUSE, PIVOT_REFINE_LITERAL = 0, 1, 2
# "refine_literal": the per-position-rescan Refine of the pages' pivot_refine
# code, prefill only (comparison)
_MODES = {"refine": PIVOT_REFINE, "reuse": PIVOT_REUSE, "refine_literal": PIVOT_REFINE_LITERAL}

#: every symbol include/pivot.h declares
EXPORTED = (
    "pivot_status_string", "pivot_candidate_count", "pivot_prefill_workspace_bytes",
    "pivot_index_prefill", "pivot_decode_workspace_bytes", "pivot_index_decode",
    "dense_index_workspace_bytes", "dense_index", "pivot_profile_enable", "pivot_profile_read",
    "pivot_sparse_attention", "pivot_index_decode_noalloc", "pivot_sparse_attention_grouped",
)

#: kernel stages reported by the stage timer (include/pivot.h)
STAGES = ("proxy", "sample_scan", "thresholds", "scan", "select", "fallback", "refine",
          "decode_scan", "decode_select")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python top_token_selection_amd/build.py)")

lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _f64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
lib.pivot_status_string.argtypes = [ctypes.c_int]
lib.pivot_status_string.restype = ctypes.c_char_p
lib.pivot_candidate_count.argtypes = [_i32, _f64, ctypes.POINTER(_i64)]
lib.pivot_candidate_count.restype = ctypes.c_int
lib.pivot_prefill_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32, _f64, _i32, _i32]
lib.pivot_prefill_workspace_bytes.restype = _sz
lib.pivot_index_prefill.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f64, _i32,
                                    _vp, _vp, _vp, _sz, _vp]
lib.pivot_index_prefill.restype = ctypes.c_int
lib.pivot_decode_workspace_bytes.argtypes = [_i32, _vp, _i32, _i32, _i32, _i32, _f64, _i32, _i32]
lib.pivot_decode_workspace_bytes.restype = _sz
lib.pivot_index_decode.argtypes = [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _i32,
                                   _vp, _vp, _vp, _sz, _vp]
lib.pivot_index_decode.restype = ctypes.c_int
lib.pivot_index_decode_noalloc.argtypes = [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _i32,
                                           _vp, _vp, _vp]
lib.pivot_index_decode_noalloc.restype = ctypes.c_int
lib.dense_index_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32]
lib.dense_index_workspace_bytes.restype = _sz
lib.dense_index.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
lib.dense_index.restype = ctypes.c_int
lib.pivot_profile_enable.argtypes = [ctypes.c_int]
lib.pivot_profile_enable.restype = ctypes.c_int
lib.pivot_profile_read.argtypes = [_vp, _vp, ctypes.c_int]
lib.pivot_profile_read.restype = ctypes.c_int
lib.pivot_sparse_attention.argtypes = [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _vp, _i32, ctypes.c_float, _vp, _vp]
lib.pivot_sparse_attention.restype = ctypes.c_int
lib.pivot_sparse_attention_grouped.argtypes = [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _vp, _i32, _i32, ctypes.c_float,
                                               _vp, _vp]
lib.pivot_sparse_attention_grouped.restype = ctypes.c_int


class PivotError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib.pivot_status_string(status).decode()} ({status})")
        self.status = status


def _check(rc: int, what: str):
    if rc != PIVOT_OK:
        raise PivotError(rc, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PIVOT_F32
    if t.dtype == torch.bfloat16:
        return PIVOT_BF16
    raise TypeError(f"q/k must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def profile_enable(on: bool = True) -> None:
    """Start (or stop) recording HIP events around every kernel stage."""
    _check(lib.pivot_profile_enable(1 if on else 0), "pivot_profile_enable")


def profile_read() -> dict:
    """{stage: (milliseconds, launches)} since the last read (waits for the
    recorded events)."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib.pivot_profile_read(ctypes.cast(ms, _vp), ctypes.cast(cnt, _vp), n), "pivot_profile_read")
    return {name: (ms[i], cnt[i]) for i, name in enumerate(STAGES) if cnt[i]}


def candidate_count(top_k: int, candidate_ratio: float) -> int:
    K = _i64()
    _check(lib.pivot_candidate_count(top_k, candidate_ratio, ctypes.byref(K)), "pivot_candidate_count")
    return K.value


def prefill_workspace_bytes(S, H, D, top_k, g, candidate_ratio=2.0, mode="refine", dtype=torch.bfloat16):
    code = PIVOT_BF16 if dtype == torch.bfloat16 else PIVOT_F32
    return int(lib.pivot_prefill_workspace_bytes(S, H, D, top_k, g, candidate_ratio, _MODES[mode], code))


def dense_workspace_bytes(S, H, D, top_k, dtype=torch.bfloat16):
    code = PIVOT_BF16 if dtype == torch.bfloat16 else PIVOT_F32
    return int(lib.dense_index_workspace_bytes(S, H, D, top_k, code))


def decode_workspace_bytes(ctx_lens, g, H, D, top_k, candidate_ratio=2.0, mode="refine", dtype=torch.bfloat16):
    ctx = torch.as_tensor(ctx_lens, dtype=torch.int64).contiguous()
    code = PIVOT_BF16 if dtype == torch.bfloat16 else PIVOT_F32
    return int(lib.pivot_decode_workspace_bytes(ctx.numel(), ctypes.c_void_p(ctx.data_ptr()), g, H, D, top_k,
                                                candidate_ratio, _MODES[mode], code))


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.device != device or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on the input device")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _per_pass_bytes(full: int, one_head: int, H: int, max_bytes):
    """Workspace that runs as many heads per pass as `max_bytes` allows."""
    if max_bytes is None or full <= max_bytes:
        return full
    per = max(1, (full - one_head) // max(1, H - 1)) if H > 1 else one_head
    fixed = one_head - per
    heads = max(1, min(H, (max_bytes - fixed) // per))
    return fixed + per * heads


def _outputs(shape, device, return_scores, out, out_scores):
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=device)
    elif out.shape != shape or out.dtype != torch.int32 or out.device != device or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 {tuple(shape)} tensor on {device}")
    sc = None
    if return_scores:
        sc = out_scores if out_scores is not None else torch.empty(shape, dtype=torch.float32, device=device)
        if sc.shape != shape or sc.dtype != torch.float32 or sc.device != device or not sc.is_contiguous():
            raise ValueError(f"out_scores must be a contiguous float32 {tuple(shape)} tensor on {device}")
    return out, sc


def index_prefill(q, k, top_k=64, g=8, candidate_ratio=2.0, mode="refine", return_scores=False,
                  workspace=None, max_workspace_bytes=None, out=None, out_scores=None):
    """PIVOT prefill indexer: int32 (S, H, top_k) (and scores). `out`,
    `out_scores` and `workspace` may be given to avoid allocations."""
    _dev(q, "q")
    _dev(k, "k")
    if q.shape != k.shape or q.dim() != 3 or q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must be (S, H, D) tensors of one dtype and device")
    S, H, D = q.shape
    code = _dtype_code(q)
    full = int(lib.pivot_prefill_workspace_bytes(S, H, D, top_k, g, candidate_ratio, _MODES[mode], code))
    if full == 0:
        # let the library name the problem
        _check(lib.pivot_index_prefill(None, None, code, S, H, D, top_k, g, candidate_ratio, _MODES[mode],
                                       None, None, None, 0, None), "pivot_index_prefill")
    one = int(lib.pivot_prefill_workspace_bytes(S, 1, D, top_k, g, candidate_ratio, _MODES[mode], code))
    ws = _workspace(_per_pass_bytes(full, one, H, max_workspace_bytes), q.device, workspace)
    out, sc = _outputs((S, H, top_k), q.device, return_scores, out, out_scores)
    _check(lib.pivot_index_prefill(_ptr(q), _ptr(k), code, S, H, D, top_k, g, candidate_ratio, _MODES[mode],
                                   _ptr(out), _ptr(sc), _ptr(ws), ws.numel(), _stream(q.device)),
           "pivot_index_prefill")
    return (out, sc) if return_scores else out


def dense_index(q, k, top_k=64, return_scores=False, workspace=None, max_workspace_bytes=None, out=None,
                out_scores=None):
    """Dense indexer (comparison): int32 (S, H, top_k) (and scores)."""
    _dev(q, "q")
    _dev(k, "k")
    if q.shape != k.shape or q.dim() != 3 or q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must be (S, H, D) tensors of one dtype and device")
    S, H, D = q.shape
    code = _dtype_code(q)
    full = int(lib.dense_index_workspace_bytes(S, H, D, top_k, code))
    if full == 0:
        _check(lib.dense_index(None, None, code, S, H, D, top_k, None, None, None, 0, None), "dense_index")
    one = int(lib.dense_index_workspace_bytes(S, 1, D, top_k, code))
    ws = _workspace(_per_pass_bytes(full, one, H, max_workspace_bytes), q.device, workspace)
    out, sc = _outputs((S, H, top_k), q.device, return_scores, out, out_scores)
    _check(lib.dense_index(_ptr(q), _ptr(k), code, S, H, D, top_k, _ptr(out), _ptr(sc), _ptr(ws), ws.numel(),
                           _stream(q.device)), "dense_index")
    return (out, sc) if return_scores else out


def index_decode(q, k_cache, ctx_lens, g, top_k=2048, candidate_ratio=2.0, mode="refine", return_scores=False,
                 workspace=None, out=None, out_scores=None):
    """PIVOT decode indexer for one MTP step of B sequences:
    q (B*g, H, D), k_cache (sum ctx, H, D), ctx_lens B host ints ->
    int32 (B*g, H, top_k) (and scores)."""
    _dev(q, "q")
    _dev(k_cache, "k_cache")
    ctx = torch.as_tensor(ctx_lens, dtype=torch.int64).cpu().contiguous()
    B = ctx.numel()
    rows, H, D = q.shape
    if rows != B * g or k_cache.dim() != 3 or k_cache.shape[1:] != (H, D) or k_cache.dtype != q.dtype:
        raise ValueError("decode shapes: q (B*g, H, D), k_cache (sum ctx, H, D), one dtype")
    if k_cache.shape[0] != int(ctx.sum()):
        raise ValueError("k_cache rows must equal the sum of ctx_lens")
    code = _dtype_code(q)
    cp = ctypes.c_void_p(ctx.data_ptr())
    need = int(lib.pivot_decode_workspace_bytes(B, cp, g, H, D, top_k, candidate_ratio, _MODES[mode], code))
    if need == 0:
        _check(lib.pivot_index_decode(None, None, code, cp, B, g, H, D, top_k, candidate_ratio, _MODES[mode],
                                      None, None, None, 0, None), "pivot_index_decode")
    ws = _workspace(need, q.device, workspace)
    out, sc = _outputs((rows, H, top_k), q.device, return_scores, out, out_scores)
    _check(lib.pivot_index_decode(_ptr(q), _ptr(k_cache), code, cp, B, g, H, D, top_k, candidate_ratio,
                                  _MODES[mode], _ptr(out), _ptr(sc), _ptr(ws), ws.numel(), _stream(q.device)),
           "pivot_index_decode")
    return (out, sc) if return_scores else out


def index_decode_noalloc(q, k_cache, ctx_lens, g, top_k=2048, candidate_ratio=2.0, mode="refine",
                         return_scores=False, out=None, out_scores=None):
    """index_decode without a workspace: the library's static device scratch
    (256 MiB per GPU) holds the intermediate arrays, and the C call
    allocates nothing (pass `out` / `out_scores` to allocate nothing here
    either). Calls that overlap on one GPU race on that scratch."""
    _dev(q, "q")
    _dev(k_cache, "k_cache")
    ctx = torch.as_tensor(ctx_lens, dtype=torch.int64).cpu().contiguous()
    B = ctx.numel()
    rows, H, D = q.shape
    if rows != B * g or k_cache.dim() != 3 or k_cache.shape[1:] != (H, D) or k_cache.dtype != q.dtype:
        raise ValueError("decode shapes: q (B*g, H, D), k_cache (sum ctx, H, D), one dtype")
    if k_cache.shape[0] != int(ctx.sum()):
        raise ValueError("k_cache rows must equal the sum of ctx_lens")
    out, sc = _outputs((rows, H, top_k), q.device, return_scores, out, out_scores)
    _check(lib.pivot_index_decode_noalloc(_ptr(q), _ptr(k_cache), _dtype_code(q), ctypes.c_void_p(ctx.data_ptr()),
                                          B, g, H, D, top_k, candidate_ratio, _MODES[mode], _ptr(out), _ptr(sc),
                                          _stream(q.device)), "pivot_index_decode_noalloc")
    return (out, sc) if return_scores else out


def sparse_attention(q, k, v, idx, scale=None, out=None, g=None):
    """Downstream sparse attention over indexer rows: float32 (S, H, D).
    softmax(scale q_i . k_c) over the entries c of idx[i, h] in [0, S) (-1 is
    padding), applied to v_c; scale defaults to D**-0.5. With g, positions
    j*g .. j*g+g-1 all attend over the row of position j*g (Reuse rows), and
    each group's rows are gathered once."""
    for name, t in (("q", q), ("k", k), ("v", v), ("idx", idx)):
        _dev(t, name)
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 3 or len({q.dtype, k.dtype, v.dtype}) != 1:
        raise ValueError("q, k and v must be (S, H, D) tensors of one dtype")
    S, H, D = q.shape
    if idx.dtype != torch.int32 or idx.dim() != 3 or tuple(idx.shape[:2]) != (S, H) or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 (S, H, top_k) tensor")
    if out is None:
        out = torch.empty((S, H, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (S, H, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 (S, H, D) tensor")
    sc = float(D) ** -0.5 if scale is None else float(scale)
    if g is not None:
        # rows shared by groups of g positions (Reuse rows): the row of each
        # group's first position serves all of its members
        _check(lib.pivot_sparse_attention_grouped(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), S, H, D, _ptr(idx),
                                                  idx.shape[2], int(g), sc, _ptr(out), _stream(q.device)),
               "pivot_sparse_attention_grouped")
        return out
    _check(lib.pivot_sparse_attention(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), S, H, D, _ptr(idx), idx.shape[2],
                                      sc, _ptr(out), _stream(q.device)), "pivot_sparse_attention")
    return out
