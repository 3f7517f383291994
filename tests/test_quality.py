"""The selection-quality measures (hierarchical_top_selection_amd.quality) against the oracle, on CPU."""
from __future__ import annotations

import numpy as np
import torch

from hierarchical_top_selection_amd import quality
from oracle import per_query
from oracle import pisa


def _inputs(seed=500, n=700, G=3, d=8):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, d))
    k[64 * 4:64 * 5] += 1.5
    q = rng.standard_normal((n, G, d)) + 0.3
    v = rng.standard_normal((n, d))
    return q, k, v


def test_recall_against_brute_force_flat_top_k():
    """Recall@K of the exact flat top-K is 1; of the hierarchical selection it is its overlap with
    the brute-force flat top-K (independent per-query routine)."""
    q, k, _ = _inputs()
    n, G, d = q.shape
    K = 3
    ts = np.array([130, 300, 511, 699])
    pyr = pisa.build_pyramid(k)
    sel, _ = pisa.route(q[ts], k, pyr, ts, K)
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    for r, t in enumerate(ts):
        flat = per_query.flat_select(k.tolist(), q[t].tolist(), int(t), K)
        got = quality.token_quality(qt[t], kt, int(t), K, {"flat": flat, "pisa": sel[r].tolist()}, 1 / np.sqrt(d))
        assert got["flat"][0] == 1.0
        want = len(set(flat).intersection(int(j) for j in sel[r] if j >= 0)) / len(flat)
        assert abs(got["pisa"][0] - want) < 1e-12


def test_mass_equals_oracle_attention_lse_ratio():
    """Mass retention of a selection is mean_h exp(LSE over its keys - LSE over all valid keys): the
    oracle's row LSE on the selection against its row LSE on every valid leaf (dense causal)."""
    q, k, v = _inputs(seed=501)
    n, G, d = q.shape
    K = 2
    ts = np.array([200, 450, 699])
    pyr = pisa.build_pyramid(k)
    sel, _ = pisa.route(q[ts], k, pyr, ts, K)
    all_leaves = np.full((len(ts), -(-n // 64)), -1)
    for r, t in enumerate(ts):
        m = t // 64 + 1
        all_leaves[r, :m] = np.arange(m)
    _, lse_sel, _ = pisa.attention(q[ts], k, v, sel, ts)
    _, lse_all, _ = pisa.attention(q[ts], k, v, all_leaves, ts)
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    for r, t in enumerate(ts):
        got = quality.token_quality(qt[t], kt, int(t), K, {"pisa": sel[r].tolist(),
                                                            "all": all_leaves[r].tolist()}, 1 / np.sqrt(d))
        want = float(np.mean(np.exp(lse_sel[r] - lse_all[r])))
        assert abs(got["pisa"][1] - want) < 1e-9
        assert abs(got["all"][1] - 1.0) < 1e-12


def test_selection_quality_aggregates_by_position():
    q, k, _ = _inputs(seed=502, n=512)
    n, G, d = q.shape
    K = 2
    pyr = pisa.build_pyramid(k)
    ts = np.arange(100, n, 37)
    sel, _ = pisa.route(q[ts], k, pyr, ts, K)
    full = np.full((1, 1, n, K), -1, dtype=np.int64)
    full[0, 0, ts] = sel
    res = quality.selection_quality(torch.from_numpy(q)[None], torch.from_numpy(k)[None, :, None],
                                    {"pisa": torch.from_numpy(full)}, ts, K, bins=4)
    r = res["pisa"]
    assert 0.0 <= r["recall"] <= 1.0 and 0.0 < r["mass"] <= 1.0
    assert len(r["recall_by_position"]) == 4 and r["recall_by_position"][0] is not None
