"""Selection quality of the block selectors on sampled query tokens.

The paper-summary page "Block Sparse Attention with Log-Linear Complexity"
(Experiments, selection quality) compares selectors by how many of the blocks
that matter they keep (Recall@K) and how much of the full attention mass the
kept blocks carry.  This module measures both for any selection on synthetic
inputs:

* reference: every causally valid leaf j of token t scored exactly, u_j = sum
  over the group's heads of the LSE of q_h . k * scale over the leaf's keys
  <= t (the leaf score of the method, applied to every leaf); its top K by
  (u desc, j asc) is the reference set;
* Recall@K(t) = |selected n reference| / |reference|;
* mass(t) = mean over the group's heads of sum over selected leaves of
  exp(LSE_{h,j} - LSE_{h,all}), the share of head h's causal softmax mass
  that falls in the selected blocks.

The reference is dense (O(t d) per token and head), so it is evaluated with
plain torch products (float32 for bf16/f32 inputs) on the device for a sample of tokens; it is a
measurement of the selectors, not part of the selection path.
"""
from __future__ import annotations

import math

import torch

LEAF = 64


def exact_leaf_lse(q: torch.Tensor, k: torch.Tensor, t: int, scale: float) -> torch.Tensor:
    """Per-head LSE of every valid leaf for token t: [G, floor(t / 64) + 1] (float32, or float64 for
    float64 inputs).

    q [G, d] the group's query heads at t, k [n, d] the group's keys (n > t).
    """
    ct = torch.promote_types(k.dtype, torch.float32)                   # float64 inputs stay float64
    keys = k[:t + 1].to(ct)
    z = (q.to(ct) @ keys.T) * scale                                    # [G, t + 1]
    m1 = t // LEAF + 1
    pad = m1 * LEAF - (t + 1)
    z = torch.nn.functional.pad(z, (0, pad), value=-math.inf)
    return torch.logsumexp(z.view(z.shape[0], m1, LEAF), dim=-1)


def token_quality(q: torch.Tensor, k: torch.Tensor, t: int, K: int, selections: dict, scale: float) -> dict:
    """Recall@K and attention-mass retention of each selection (name -> leaf ids) for token t."""
    lse = exact_leaf_lse(q, k, t, scale)                               # [G, M]
    u = lse.sum(dim=0)
    M = u.shape[0]
    order = torch.sort(-u, stable=True).indices                        # (u desc, j asc)
    ref = set(order[:min(K, M)].tolist())
    total = torch.logsumexp(lse, dim=-1)                               # [G]
    out = {}
    for name, sel in selections.items():
        chosen = [int(j) for j in sel if 0 <= int(j) < M]
        if chosen:
            idx = torch.tensor(chosen, device=u.device)
            mass = torch.exp(torch.logsumexp(lse[:, idx], dim=-1) - total).mean().item()
        else:
            mass = 0.0
        out[name] = (len(ref.intersection(chosen)) / len(ref), mass)
    return out


def selection_quality(q: torch.Tensor, k: torch.Tensor, sels: dict, ts, K: int, kvh: int = 0, b: int = 0,
                      scale: float | None = None, bins: int = 4) -> dict:
    """Mean Recall@K and mass retention per method over tokens ts, overall and per position bin.

    q [B, N, Hq, d], k [B, N, Hkv, d]; sels maps a method name to its selection tensor
    [B, Hkv, N, K] (ascending ids, -1 padded).
    """
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qg = q[b, :, kvh * G:(kvh + 1) * G]
    kk = k[b, :, kvh]
    rows = {name: s[b, kvh].cpu() for name, s in sels.items()}
    acc = {name: [[0.0, 0.0, 0] for _ in range(bins)] for name in sels}
    for t in ts:
        t = int(t)
        res = token_quality(qg[t], kk, t, K, {name: rows[name][t].tolist() for name in sels}, scale)
        bi = min(bins - 1, t * bins // N)
        for name, (rec, mass) in res.items():
            acc[name][bi][0] += rec
            acc[name][bi][1] += mass
            acc[name][bi][2] += 1
    out = {}
    for name, per_bin in acc.items():
        n = sum(c for _, _, c in per_bin)
        out[name] = {
            "recall": sum(r for r, _, _ in per_bin) / max(n, 1),
            "mass": sum(m for _, m, _ in per_bin) / max(n, 1),
            "recall_by_position": [r / c if c else None for r, _, c in per_bin],
            "mass_by_position": [m / c if c else None for _, m, c in per_bin],
        }
    return out
