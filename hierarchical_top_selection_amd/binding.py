"""Python binding of libpisa.so: the C ABI of include/pisa.h with torch tensors.

Argument marshalling only: every step of the path runs in the HIP kernels of
the shared library.  The library is loaded on first use; if it has not been
built, or cannot be loaded, every call raises -- there is no fallback.

Tensors (device, contiguous in the head_dim axis):
  q  [B, N, Hq, d]   k, v  [B, N, Hkv, d]   bfloat16 or float32
  pyramid            float32 [B, Hkv, pyramid_nodes(capacity), d]
  selection          int32 [B, Hkv, N, K], ascending leaf ids, -1 padded
Work is enqueued on torch's current stream of the tensors' device.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpisa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pisa.h")

LEAF = 64
FANOUT = 2
PISA_F32, PISA_BF16 = 0, 1


class PisaCfg(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("fanout", ctypes.c_int32), ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("score", ctypes.c_int32)]


SCORES = {"lse": 0, "mean": 1, "mean_var": 2}   # PISA, PISA-1, PISA-2 candidate scores


class PisaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


_P = ctypes.POINTER
_SIGNATURES = {
    "pisa_abi_version": (ctypes.c_int, []),
    "pisa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pisa_last_hip_error": (ctypes.c_int, []),
    "pisa_stage_events": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "pisa_pyramid_nodes": (ctypes.c_int64, [ctypes.c_int32]),
    "pisa_pyramid_bytes": (ctypes.c_size_t, [_P(PisaCfg), ctypes.c_int32]),
    "pisa_build_pyramid": (ctypes.c_int, [_P(PisaCfg), PisaTensor, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "pisa_select_workspace_bytes": (ctypes.c_size_t, [_P(PisaCfg)]),
    "pisa_select_blocks": (ctypes.c_int, [_P(PisaCfg), PisaTensor, PisaTensor, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pisa_flat_workspace_bytes": (ctypes.c_size_t, [_P(PisaCfg)]),
    "pisa_select_flat": (ctypes.c_int, [_P(PisaCfg), PisaTensor, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pisa_attn_workspace_bytes": (ctypes.c_size_t, [_P(PisaCfg)]),
    "pisa_sparse_attn_fwd": (ctypes.c_int, [_P(PisaCfg), PisaTensor, PisaTensor, PisaTensor, ctypes.c_void_p,
                                            PisaTensor, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "pisa_sparse_attn_fwd_noalloc": (ctypes.c_int, [_P(PisaCfg), PisaTensor, PisaTensor, PisaTensor,
                                                    ctypes.c_void_p, PisaTensor, ctypes.c_int, ctypes.c_void_p,
                                                    ctypes.c_void_p]),
    "pisa_attn_bwd_workspace_bytes": (ctypes.c_size_t, [_P(PisaCfg)]),
    "pisa_sparse_attn_bwd": (ctypes.c_int, [_P(PisaCfg), PisaTensor, PisaTensor, PisaTensor, ctypes.c_void_p,
                                            PisaTensor, PisaTensor, ctypes.c_int, ctypes.c_void_p, PisaTensor,
                                            PisaTensor, PisaTensor, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "pisa_decode_step": (ctypes.c_int, [_P(PisaCfg), ctypes.c_int32, PisaTensor, PisaTensor, PisaTensor,
                                        PisaTensor, PisaTensor, ctypes.c_void_p, ctypes.c_void_p, PisaTensor,
                                        ctypes.c_int, ctypes.c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it is missing or incomplete)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m hierarchical_top_selection_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/pisa.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(pisa_\w+)\s*\(", text)))


def _check(name: str, status: int) -> None:
    if status != 0:
        msg = lib().pisa_status_string(status).decode()
        raise RuntimeError(f"{name} failed: {msg} (status {status}, hip error {lib().pisa_last_hip_error()})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PISA_BF16
    if t.dtype == torch.float32:
        return PISA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: expected bfloat16 or float32")


def _tensor(t: torch.Tensor, token_axis: bool = True) -> PisaTensor:
    if t.stride(-1) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    if token_axis:
        sb, st, sh = t.stride(0), t.stride(1), t.stride(2)
    else:
        sb, st, sh = t.stride(0), 0, t.stride(1)
    return PisaTensor(t.data_ptr(), sb, st, sh)


def _extent(t: torch.Tensor) -> tuple[int, int]:
    """Byte range [start, end) that a (possibly strided) tensor's elements span."""
    if t.numel() == 0:
        return t.data_ptr(), t.data_ptr()
    last = sum((size - 1) * stride for size, stride in zip(t.shape, t.stride()))
    return t.data_ptr(), t.data_ptr() + (last + 1) * t.element_size()


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    (a0, a1), (b0, b1) = _extent(a), _extent(b)
    return a0 < b1 and b0 < a1


def _expect(name: str, t: torch.Tensor, shape, dtype=None, device=None) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ws_bytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_STAGE_ARRAY = []   # keeps the handle array of stage_events alive until the next call has used it


def stage_events(events) -> None:
    """Hands timing-enabled torch.cuda.Event objects to the next binding call on this thread: the
    library records events[i] on its stream right after it enqueues its i-th kernel."""
    handles = []
    for e in events:
        if not e.cuda_event:                  # torch creates the event on its first record
            e.record()
        handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    _STAGE_ARRAY[:] = [arr]
    _check("pisa_stage_events", lib().pisa_stage_events(ctypes.cast(arr, ctypes.c_void_p), len(handles)))


def make_cfg(batch: int, seq_len: int, n_q_heads: int, n_kv_heads: int, head_dim: int, top_k: int,
             dtype: torch.dtype, scale: float = 0.0, score: str = "lse") -> PisaCfg:
    code = PISA_BF16 if dtype == torch.bfloat16 else PISA_F32
    if score not in SCORES:
        raise ValueError(f"score must be one of {sorted(SCORES)}")
    return PisaCfg(batch, seq_len, n_q_heads, n_kv_heads, head_dim, LEAF, FANOUT, top_k, code, scale, SCORES[score])


def pyramid_nodes(capacity: int) -> int:
    return int(lib().pisa_pyramid_nodes(capacity))


def _cfg_from(q_or_none, k: torch.Tensor, top_k: int, scale: float, seq_len: int | None = None) -> PisaCfg:
    B, N, Hkv, d = k.shape
    Hq = q_or_none.shape[2] if q_or_none is not None else Hkv
    cfg = make_cfg(B, N if seq_len is None else seq_len, Hq, Hkv, d, top_k, k.dtype, scale)
    _dtype_code(k)
    return cfg


def build_pyramid(k: torch.Tensor, n: int | None = None, capacity: int | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Mean-pooled key pyramid of k [B, >=n, Hkv, d] for length n, laid out for `capacity` keys."""
    B, N, Hkv, d = k.shape
    n = N if n is None else n
    capacity = n if capacity is None else capacity
    cfg = _cfg_from(None, k, 1, 0.0, seq_len=capacity)
    nodes = pyramid_nodes(capacity)
    if out is None:
        out = torch.empty((B, Hkv, nodes, d), dtype=torch.float32, device=k.device)
    elif out.shape != (B, Hkv, nodes, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("pyramid buffer has the wrong shape, dtype or layout")
    _check("pisa_build_pyramid", lib().pisa_build_pyramid(ctypes.byref(cfg), _tensor(k), n, capacity,
                                                         ctypes.c_void_p(out.data_ptr()), _stream(k)))
    return out


def select_workspace_bytes(cfg: PisaCfg) -> int:
    return int(lib().pisa_select_workspace_bytes(ctypes.byref(cfg)))


def select_blocks(q: torch.Tensor, k: torch.Tensor, pyr: torch.Tensor, top_k: int, scale: float = 0.0,
                  workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  return_scores: bool = False, score: str = "lse"):
    """Hierarchical top-K leaf selection: int32 [B, Hkv, N, K] (and float32 scores if asked).

    ``score``: "lse" (the method), "mean" or "mean_var" (the PISA-1 / PISA-2 variants).
    """
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    _expect("k", k, (B, N, Hkv, d), q.dtype, q.device)
    _expect("pyramid", pyr, (B, Hkv, pyramid_nodes(N), d), torch.float32, q.device)
    cfg = _cfg_from(q, k, top_k, scale)
    cfg.score = SCORES[score]
    need = select_workspace_bytes(cfg)
    if workspace is None or _ws_bytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hkv, N, top_k), dtype=torch.int32, device=q.device)
    _expect("out", out, (B, Hkv, N, top_k), torch.int32, q.device)
    if not out.is_contiguous() or not pyr.is_contiguous():
        raise ValueError("the selection and the pyramid must be contiguous")
    scores = torch.empty((B, Hkv, N, top_k), dtype=torch.float32, device=q.device) if return_scores else None
    _check("pisa_select_blocks", lib().pisa_select_blocks(
        ctypes.byref(cfg), _tensor(q), _tensor(k), ctypes.c_void_p(pyr.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(scores.data_ptr() if scores is not None else 0),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(_ws_bytes(workspace)), _stream(q)))
    return (out, scores) if return_scores else out


def flat_workspace_bytes(cfg: PisaCfg) -> int:
    return int(lib().pisa_flat_workspace_bytes(ctypes.byref(cfg)))


def select_flat(q: torch.Tensor, pyr: torch.Tensor, n_kv_heads: int, top_k: int, scale: float = 0.0,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                return_scores: bool = False):
    """Single-level (flat) top-K leaf selection by mean-key scores: int32 [B, Hkv, N, K] (and scores)."""
    B, N, Hq, d = q.shape
    _dtype_code(q)
    _expect("pyramid", pyr, (B, n_kv_heads, pyramid_nodes(N), d), torch.float32, q.device)
    cfg = make_cfg(B, N, Hq, n_kv_heads, d, top_k, q.dtype, scale)
    need = flat_workspace_bytes(cfg)
    if workspace is None or _ws_bytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, n_kv_heads, N, top_k), dtype=torch.int32, device=q.device)
    _expect("out", out, (B, n_kv_heads, N, top_k), torch.int32, q.device)
    if not out.is_contiguous() or not pyr.is_contiguous():
        raise ValueError("the selection and the pyramid must be contiguous")
    scores = torch.empty((B, n_kv_heads, N, top_k), dtype=torch.float32, device=q.device) if return_scores else None
    _check("pisa_select_flat", lib().pisa_select_flat(
        ctypes.byref(cfg), _tensor(q), ctypes.c_void_p(pyr.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(scores.data_ptr() if scores is not None else 0),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(_ws_bytes(workspace)), _stream(q)))
    return (out, scores) if return_scores else out


def attn_workspace_bytes(cfg: PisaCfg) -> int:
    return int(lib().pisa_attn_workspace_bytes(ctypes.byref(cfg)))


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, scale: float = 0.0,
                    out: torch.Tensor | None = None, return_lse: bool = False, out_dtype: torch.dtype | None = None,
                    workspace: torch.Tensor | None = None):
    """Attention over the selected blocks: o [B, N, Hq, d] (and row LSE [B, Hq, N] if asked).

    The output is float32 or bfloat16 (default: q's dtype, or the dtype of ``out``).
    """
    B, N, Hq, d = q.shape
    top_k = sel.shape[-1]
    Hkv = k.shape[2]
    _expect("k", k, (B, N, Hkv, d), q.dtype, q.device)
    _expect("v", v, (B, N, Hkv, d), q.dtype, q.device)
    cfg = _cfg_from(q, k, top_k, scale)
    if sel.dtype != torch.int32 or not sel.is_contiguous() or sel.shape != (B, Hkv, N, top_k):
        raise ValueError("selection must be a contiguous int32 [B, Hkv, N, K] tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _expect("out", out, q.shape, out_dtype, q.device)
    _dtype_code(out)
    if any(_overlap(out, x) for x in (q, k, v, sel)):
        raise ValueError("out must not overlap q, k, v or the selection")
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if return_lse else None
    need = attn_workspace_bytes(cfg)
    if need and (workspace is None or _ws_bytes(workspace) < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_len = (workspace.data_ptr(), _ws_bytes(workspace)) if need else (0, 0)
    _check("pisa_sparse_attn_fwd", lib().pisa_sparse_attn_fwd(
        ctypes.byref(cfg), _tensor(q), _tensor(k), _tensor(v), ctypes.c_void_p(sel.data_ptr()),
        _tensor(out), _dtype_code(out), ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
        ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_len), _stream(q)))
    return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 128 << 20       # PISA_NOALLOC_SCRATCH_BYTES


def sparse_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor,
                            out: torch.Tensor, lse_out: torch.Tensor | None = None, scale: float = 0.0):
    """`sparse_attn_fwd` through the allocation-free entry point: the caller passes the output (and
    optionally the row LSE [B, Hq, N] float32) and the workspace is the library's fixed device
    array; nothing is allocated here either."""
    B, N, Hq, d = q.shape
    top_k = sel.shape[-1]
    Hkv = k.shape[2]
    _expect("k", k, (B, N, Hkv, d), q.dtype, q.device)
    _expect("v", v, (B, N, Hkv, d), q.dtype, q.device)
    cfg = _cfg_from(q, k, top_k, scale)
    if sel.dtype != torch.int32 or not sel.is_contiguous() or sel.shape != (B, Hkv, N, top_k):
        raise ValueError("selection must be a contiguous int32 [B, Hkv, N, K] tensor")
    _expect("out", out, q.shape, None, q.device)
    _dtype_code(out)
    if any(_overlap(out, x) for x in (q, k, v, sel)):
        raise ValueError("out must not overlap q, k, v or the selection")
    if lse_out is not None:
        _expect("lse_out", lse_out, (B, Hq, N), torch.float32, q.device)
        if not lse_out.is_contiguous():
            raise ValueError("lse_out must be contiguous")
    _check("pisa_sparse_attn_fwd_noalloc", lib().pisa_sparse_attn_fwd_noalloc(
        ctypes.byref(cfg), _tensor(q), _tensor(k), _tensor(v), ctypes.c_void_p(sel.data_ptr()),
        _tensor(out), _dtype_code(out), ctypes.c_void_p(lse_out.data_ptr() if lse_out is not None else 0),
        _stream(q)))
    return out


def attn_bwd_workspace_bytes(cfg: PisaCfg) -> int:
    return int(lib().pisa_attn_bwd_workspace_bytes(ctypes.byref(cfg)))


def sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, o: torch.Tensor,
                    row_lse: torch.Tensor, dout: torch.Tensor, scale: float = 0.0, workspace: torch.Tensor | None = None,
                    dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Gradients (dq [B, N, Hq, d], dk and dv [B, N, Hkv, d], float32) of `sparse_attn_fwd` with the
    selections held fixed; o and row_lse are that call's output and row LSE, dout the upstream
    gradient (same dtype as o)."""
    B, N, Hq, d = q.shape
    top_k = sel.shape[-1]
    cfg = _cfg_from(q, k, top_k, scale)
    if sel.dtype != torch.int32 or not sel.is_contiguous() or sel.shape != (B, k.shape[2], N, top_k):
        raise ValueError("selection must be a contiguous int32 [B, Hkv, N, K] tensor")
    if dout.dtype != o.dtype or dout.shape != o.shape or o.shape != q.shape:
        raise ValueError("o and dout must have q's shape and one dtype")
    if row_lse.dtype != torch.float32 or not row_lse.is_contiguous() or row_lse.shape != (B, Hq, N):
        raise ValueError("row_lse must be a contiguous float32 [B, Hq, N] tensor")
    _expect("k", k, (B, N, k.shape[2], d), q.dtype, q.device)
    _expect("v", v, k.shape, q.dtype, q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    for name, x, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _expect(name, x, ref.shape, torch.float32, q.device)
    need = attn_bwd_workspace_bytes(cfg)
    if need == 0:
        raise RuntimeError("pisa_sparse_attn_bwd: unsupported configuration")
    if workspace is None or _ws_bytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check("pisa_sparse_attn_bwd", lib().pisa_sparse_attn_bwd(
        ctypes.byref(cfg), _tensor(q), _tensor(k), _tensor(v), ctypes.c_void_p(sel.data_ptr()), _tensor(o),
        _tensor(dout), _dtype_code(dout), ctypes.c_void_p(row_lse.data_ptr()), _tensor(dq), _tensor(dk), _tensor(dv),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(_ws_bytes(workspace)), _stream(q)))
    return dq, dk, dv


def decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, pyr: torch.Tensor, n_ctx: int, top_k: int, scale: float = 0.0,
                out: torch.Tensor | None = None, sel_out: torch.Tensor | None = None,
                out_dtype: torch.dtype | None = None, score: str = "lse"):
    """One decode step for every sequence: q [B, Hq, d], k_new/v_new [B, Hkv, d], caches [B, cap, Hkv, d].

    Appends at position n_ctx, updates the pyramid in place and returns (o [B, Hq, d], sel [B, Hkv, K]).
    """
    B, cap, Hkv, d = k_cache.shape
    Hq = q.shape[1]
    dt, dev = k_cache.dtype, k_cache.device
    _dtype_code(k_cache)
    _expect("q", q, (B, Hq, d), dt, dev)
    _expect("k_new", k_new, (B, Hkv, d), dt, dev)
    _expect("v_new", v_new, (B, Hkv, d), dt, dev)
    _expect("v_cache", v_cache, k_cache.shape, dt, dev)
    _expect("pyramid", pyr, (B, Hkv, pyramid_nodes(cap), d), torch.float32, dev)
    if not pyr.is_contiguous():
        raise ValueError("the pyramid must be contiguous")
    cfg = make_cfg(B, cap, Hq, Hkv, d, top_k, dt, scale, score)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _expect("out", out, q.shape, out_dtype, dev)
    _dtype_code(out)
    if sel_out is None:
        sel_out = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=q.device)
    _expect("sel_out", sel_out, (B, Hkv, top_k), torch.int32, dev)
    if not sel_out.is_contiguous():
        raise ValueError("sel_out must be contiguous")
    _check("pisa_decode_step", lib().pisa_decode_step(
        ctypes.byref(cfg), n_ctx, _tensor(q, False), _tensor(k_new, False), _tensor(v_new, False),
        _tensor(k_cache), _tensor(v_cache), ctypes.c_void_p(pyr.data_ptr()), ctypes.c_void_p(sel_out.data_ptr()),
        _tensor(out, False), _dtype_code(out), _stream(q)))
    return out, sel_out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
