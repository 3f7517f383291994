"""Routing with the float16 pre-filter (the default for bf16 inputs, every score) keeps exactly
the candidates that routing keeps when it scores every candidate from the full split rows
(PISA_ROUTE_EXACT=1 in the environment).  A child process with the variable set routes the same
inputs; the leaf candidates that routing leaves in the workspace and the final selections must agree
bit for bit on every token, over several lengths, group sizes, K and head dims, on N(0,1) inputs
with planted blocks (a key direction shared with the queries, which makes scores close).
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gpu_harness as H
from hierarchical_top_selection_amd import binding

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (B, N, Hq, Hkv, d, K, planted blocks per 1024 leaves, key shift, seed, regime)
# Regimes beyond N(0,1): "ties" (every key the same, so every score ties and the lower index
# decides), "huge" (keys of order 1e6: summaries beyond the float16 range, clamped, so the bounds
# must send those candidates to the split rows), "tiny" (keys of order 1e-6: float16 subnormal
# summaries) and "subq" (queries with elements below the float16 normal range, so q - q_lo != 0).
CASES = [
    (1, 262144, 16, 1, 128, 16, 5, 2.0, 1, "normal"),
    (2, 32768, 32, 2, 128, 32, 8, 2.0, 2, "normal"),
    (1, 65536, 16, 1, 128, 8, 16, 3.0, 3, "normal"),
    (2, 20000, 16, 2, 64, 12, 8, 2.0, 4, "normal"),
    (1, 9000, 8, 8, 128, 5, 4, 1.0, 5, "normal"),
    (3, 3000, 4, 2, 128, 3, 0, 0.0, 6, "normal"),
    (1, 5000, 16, 16, 64, 1, 32, 4.0, 7, "normal"),
    (1, 6000, 16, 1, 128, 8, 0, 0.0, 8, "ties"),
    (1, 6000, 16, 1, 128, 8, 8, 2.0, 9, "huge"),
    (1, 6000, 16, 1, 128, 8, 8, 2.0, 10, "tiny"),
    (1, 6000, 8, 1, 64, 4, 8, 2.0, 11, "subq"),
]


def draw(case):
    B, N, Hq, Hkv, d, K, plant, shift, seed, regime = case
    gen = torch.Generator(device=H.DEV)
    gen.manual_seed(seed)
    u = torch.randn(d, generator=gen, device=H.DEV)
    u = u / u.norm()
    q = torch.randn((B, N, Hq, d), generator=gen, device=H.DEV) + u
    k = torch.randn((B, N, Hkv, d), generator=gen, device=H.DEV)
    m1 = -(-N // 64)
    n_plant = round(plant * m1 / 1024)
    for b in range(B):
        for h in range(Hkv):
            for j in torch.randperm(m1, generator=gen, device=H.DEV)[:n_plant].tolist():
                k[b, 64 * j:64 * j + 64, h] += shift * u
    if regime == "ties":
        k = torch.full_like(k, 0.375)
    elif regime == "huge":
        k = k * 1e6
    elif regime == "tiny":
        k = k * 1e-6
    elif regime == "subq":
        q = torch.where(torch.rand(q.shape, generator=gen, device=H.DEV) < 0.05, q * 1e-6, q)
    return q.to(torch.bfloat16), k.to(torch.bfloat16)


# the score variants (PISA-1 / PISA-2) on a subset of the cases
VARIANT_CASES = (1, 4, 7, 8, 9, 10)


def runs():
    for i in range(len(CASES)):
        yield i, "lse"
    for i in VARIANT_CASES:
        for score in ("mean", "mean_var"):
            yield i, score


def run_all() -> dict:
    out = {}
    for i, score in runs():
        case = CASES[i]
        B, N, Hq, Hkv, d, K = case[:6]
        q, k = draw(case)
        pyr = binding.build_pyramid(k)
        cfg = binding.make_cfg(B, N, Hq, Hkv, d, K, q.dtype)
        ws = torch.empty(binding.select_workspace_bytes(cfg), dtype=torch.uint8, device=H.DEV)
        sel = binding.select_blocks(q, k, pyr, K, workspace=ws, score=score)
        torch.cuda.synchronize()
        slots = B * Hkv * N * 2 * K
        out[f"cand{i}_{score}"] = ws[:slots * 4].view(torch.int32).cpu().numpy()
        out[f"sel{i}_{score}"] = sel.cpu().numpy()
        del q, k, pyr, ws, sel
        torch.cuda.empty_cache()
    return out


def child(path: str) -> None:
    np.savez(path, **run_all())


def test_prefilter_keeps_what_exact_routing_keeps(tmp_path):
    here = run_all()
    out = str(tmp_path / "exact.npz")
    env = dict(os.environ, PISA_ROUTE_EXACT="1")
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]; "
            f"import test_gpu_route_prefilter as m; m.child({out!r})")
    H.log("[route pre-filter] child process with PISA_ROUTE_EXACT=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    there = np.load(out)
    for i, score in runs():
        case = CASES[i]
        for name in (f"cand{i}_{score}", f"sel{i}_{score}"):
            diff = int((here[name] != there[name]).sum())
            H.log(f"[route pre-filter] case {case[:6]} {case[9]} {score} {name.split(str(i))[0]}: {diff} differing entries")
            assert diff == 0, (case, score, name)
