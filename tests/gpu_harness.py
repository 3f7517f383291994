"""Helpers for the GPU parity tests: seeded inputs on both sides, oracle runs on
sampled tokens, and the comparison rules.

Comparison rules (from the acceptance criteria of the hot path):
  * selections are compared as sets per (b, kvh, token); a difference is
    allowed only where the oracle's K-th vs (K+1)-th score gap at some scored
    level is below 1e-3, and such cases must stay under 0.1% of the queries a
    test compares, pooled over all its (b, kvh) units (so a test that compares
    fewer than 1000 queries allows none);
  * attention is compared against the oracle's attention over the ORACLE's
    selection, which is fed to the GPU kernel as its input: max-abs <= 1e-2 and
    relative L2 <= 5e-3 for bf16 inputs with fp32 accumulation (1e-4 / 1e-5 for
    fp32 inputs).
No value computed by the GPU path is ever fed into the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W
from oracle import pisa as oracle

GAP_LIMIT = 1e-3
DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(w: W.Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def to_device(x: np.ndarray, w: W.Workload) -> torch.Tensor:
    """Host values in the workload dtype (float32 values, or uint16 bf16 patterns) -> device tensor."""
    if w.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    bits = x if x.dtype == np.uint16 else W.round_bf16_bits(x)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_values(x: np.ndarray) -> np.ndarray:
    """Storage array (float32 or uint16 bf16 patterns) -> float32 values."""
    return W.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def sample_tokens(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted sample of positions: edges and leaf boundaries plus uniform draws."""
    fixed = {0, 1, 62, 63, 64, 65, 127, 128, n - 1, n - 2, n - 64, n - 65, n // 2}
    rng = np.random.default_rng(seed)
    extra = rng.choice(n, size=min(n, count), replace=False)
    return np.array(sorted(t for t in fixed.union(extra.tolist()) if 0 <= t < n), dtype=np.int64)


def run_gpu_prefill(w: W.Workload, q: np.ndarray, k: np.ndarray, v: np.ndarray, top_k: int | None = None):
    """Pyramid, selection (+ scores) and attention on the GPU for host arrays [B, N, H, d]."""
    K = w.top_k if top_k is None else top_k
    qd, kd, vd = to_device(q, w), to_device(k, w), to_device(v, w)
    pyr = binding.build_pyramid(kd)
    sel, sel_u = binding.select_blocks(qd, kd, pyr, K, return_scores=True)
    o, lse = binding.sparse_attn_fwd(qd, kd, vd, sel, return_lse=True, out_dtype=torch.float32)
    o_native = binding.sparse_attn_fwd(qd, kd, vd, sel)          # output in the input dtype
    torch.cuda.synchronize()
    return {"q": qd, "k": kd, "v": vd, "pyr": pyr, "sel": sel, "sel_u": sel_u, "o": o, "lse": lse,
            "o_native": o_native}


def oracle_prefill(w: W.Workload, q, k, v, b: int, kvh: int, ts: np.ndarray, top_k: int | None = None):
    K = w.top_k if top_k is None else top_k
    G = w.group
    qg = host_values(q[b, :, kvh * G:(kvh + 1) * G, :]).astype(np.float64)
    kk = host_values(k[b, :, kvh]).astype(np.float64)
    vv = host_values(v[b, :, kvh]).astype(np.float64)
    return oracle.prefill(qg, kk, vv, K, ts=ts)


def compare_selection(gpu_sel: np.ndarray, ora_sel: np.ndarray, gap: np.ndarray, label: str):
    """Returns (n_mismatch, mask of agreeing rows); asserts the boundary rule."""
    agree = np.all(gpu_sel == ora_sel, axis=1)
    bad = np.nonzero(~agree)[0]
    for r in bad:
        assert gap[r] < GAP_LIMIT, f"{label}: row {r} differs with oracle gap {gap[r]:.3g}: " \
                                   f"gpu {gpu_sel[r].tolist()} oracle {ora_sel[r].tolist()}"
    return len(bad), agree


def assert_mismatch_budget(n_bad: int, n_total: int, label: str) -> None:
    """Boundary mismatches pooled over every query one test compares must stay under 0.1%."""
    allowed = int(0.001 * n_total)
    log(f"{label}: {n_bad} boundary mismatches of {n_total} queries (allowed {allowed})")
    assert n_bad <= allowed, f"{label}: {n_bad} boundary mismatches of {n_total} queries"


def attn_errors(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)) if got.size else 0.0
    return max_abs, rel_l2


def attn_tolerance(w: W.Workload):
    """(max-abs, relative L2) gates for float32 outputs."""
    return (1e-4, 1e-5) if w.dtype == "f32" else (1e-2, 5e-3)


def assert_bf16_output(got: np.ndarray, want: np.ndarray, label: str, abs_gate: float = 1e-2) -> None:
    """bfloat16 outputs: the fp32 gates plus half a bf16 ulp of the exact value (<= |x| / 256)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want) - np.abs(want) / 256.0
    assert err.size == 0 or err.max() <= abs_gate, (label, "bf16 output", float(err.max()))
    _, rl = attn_errors(got, want)
    assert rl <= 5e-3, (label, "bf16 output rel-L2", rl)
