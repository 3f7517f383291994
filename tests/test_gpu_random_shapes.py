"""GPU parity over seeded random shapes: batch, length (ragged and exact multiples of 64), KV heads,
group size, head dim, K (up to 32, beyond the number of leaves as well), input dtype and candidate
score, drawn once from a fixed seed so the list is the same on every run.  Every token of every
prefill case goes through the oracle comparison of the parity tests (pyramid, selections under the
boundary rule, leaf scores, attention end to end and on the oracle's own selection; the variant
cases compare selections and leaf scores); every step of every decode case is compared with the
decode oracle (selection, output, and the incremental pyramid against a rebuild); every gradient of
every backward case is compared with the oracle's (the backward tests' tolerances); every token of
every flat-selection case is compared with the oracle's single-level selection.  The boundary
mismatches are pooled over all cases of a test against the 0.1% budget.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_harness as H
from hierarchical_top_selection_amd import workloads as W
from test_gpu_backward import check_full
from test_gpu_flat import check_flat
from test_gpu_parity import check_prefill, run_decode
from test_gpu_variants import check_variant

pytestmark = pytest.mark.gpu


def cases(count: int = 48):
    rng = np.random.default_rng(2024)
    out = []
    for i in range(count):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        n = int(rng.choice([int(rng.integers(1, 3000)), 64 * int(rng.integers(1, 45))]))
        b = int(rng.integers(1, 4)) if n * hkv <= 2000 else 1
        d = int(rng.choice([64, 128]))
        k = int(rng.integers(1, 33))
        dtype = "f32" if i % 6 == 5 else "bf16"
        score = ("lse", "lse", "mean", "mean_var")[i % 4]
        out.append(dict(batch=b, seq_len=n, n_kv_heads=hkv, n_q_heads=g * hkv, head_dim=d, top_k=k, dtype=dtype,
                        seed=300 + i, score=score))
    return out


def test_random_shapes_pooled_budget():
    counts = []
    for i, c in enumerate(cases()):
        score = c.pop("score")
        w = W.WORKLOADS["prefill_n4096"].with_(name=f"rand{i}", **c)
        label = (f"rand{i}_b{w.batch}_n{w.seq_len}_hkv{w.n_kv_heads}_g{w.group}_d{w.head_dim}_k{w.top_k}_"
                 f"{w.dtype}_{score}")
        if score == "lse":
            check_prefill(w, label, counts=counts)
        else:
            check_variant(w, score, label, counts=counts)
    n_bad = sum(c[0] for c in counts)
    n_total = sum(c[1] for c in counts)
    H.assert_mismatch_budget(n_bad, n_total, "random shapes")


def decode_cases(count: int = 40):
    rng = np.random.default_rng(2025)
    out = []
    for i in range(count):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        k = int(rng.integers(1, min(16, 128 // g) + 1))          # G * 2K <= 256 (leaf logits on chip)
        d = int(rng.choice([64, 128]))
        n0 = int(rng.choice([int(rng.integers(1, 3000)), 64 * int(rng.integers(1, 40)) - 1]))
        steps = int(rng.integers(5, 81))
        b = int(rng.integers(1, 3))
        dtype = "f32" if i % 5 == 4 else "bf16"
        out.append((dict(n_kv_heads=hkv, n_q_heads=g * hkv, top_k=k, head_dim=d, decode_steps=steps, dtype=dtype,
                         seed=400 + i), b, n0, steps))
    return out


def test_random_decode_shapes_pooled_budget():
    counts = []
    for i, (c, b, n0, steps) in enumerate(decode_cases()):
        w = W.WORKLOADS["decode_b64_ctx131072"].with_(name=f"dec_rand{i}", **c)
        label = (f"dec_rand{i}_b{b}_ctx{n0}_s{steps}_hkv{w.n_kv_heads}_g{w.group}_d{w.head_dim}_k{w.top_k}_"
                 f"{w.dtype}")
        run_decode(w, list(range(b)), n0, steps, label, counts=counts)
    n_bad = sum(c[0] for c in counts)
    n_total = sum(c[1] for c in counts)
    H.assert_mismatch_budget(n_bad, n_total, "random decode shapes")


def backward_cases(count: int = 16):
    rng = np.random.default_rng(2026)
    out = []
    for i in range(count):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        n = int(rng.choice([int(rng.integers(1, 2000)), 64 * int(rng.integers(1, 30))]))
        b = int(rng.integers(1, 3)) if n * hkv <= 1500 else 1
        d = int(rng.choice([64, 128]))
        k = int(rng.integers(1, 33))
        out.append((dict(batch=b, seq_len=n, n_kv_heads=hkv, n_q_heads=g * hkv, head_dim=d, seed=500 + i), k,
                    ("route", "random")[i % 2], (torch.float32, torch.bfloat16)[(i // 2) % 2]))
    return out


def test_random_backward_shapes():
    for i, (c, k, selection, grad_dtype) in enumerate(backward_cases()):
        w = W.WORKLOADS["prefill_n4096"].with_(name=f"bwd_rand{i}", **c)
        label = (f"bwd_rand{i}_b{w.batch}_n{w.seq_len}_hkv{w.n_kv_heads}_g{w.group}_d{w.head_dim}_k{k}_{selection}_"
                 f"{str(grad_dtype).split('.')[-1]}")
        check_full(w, k, label, selection=selection, grad_dtype=grad_dtype)


def flat_cases(count: int = 16):
    rng = np.random.default_rng(2027)
    out = []
    for i in range(count):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        n = int(rng.choice([int(rng.integers(1, 3000)), 64 * int(rng.integers(1, 45))]))
        b = int(rng.integers(1, 3)) if n * hkv <= 2000 else 1
        out.append((dict(batch=b, seq_len=n, n_kv_heads=hkv, n_q_heads=g * hkv, head_dim=int(rng.choice([64, 128])),
                         dtype="f32" if i % 5 == 4 else "bf16", seed=600 + i), int(rng.integers(1, 17))))
    return out


def test_random_flat_shapes_pooled_budget():
    counts = []
    for i, (c, k) in enumerate(flat_cases()):
        w = W.WORKLOADS["prefill_n4096"].with_(name=f"flat_rand{i}", **c)
        label = f"flat_rand{i}_b{w.batch}_n{w.seq_len}_hkv{w.n_kv_heads}_g{w.group}_d{w.head_dim}_k{k}_{w.dtype}"
        check_flat(w, k, label, counts=counts)
    n_bad = sum(c[0] for c in counts)
    n_total = sum(c[1] for c in counts)
    H.assert_mismatch_budget(n_bad, n_total, "random flat shapes")
