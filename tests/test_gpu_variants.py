"""GPU parity of the PISA-1 (mean) and PISA-2 (mean + var/2) candidate scores against the oracle.

Same rules as the main parity tests: selections bit-exact except where the oracle's K-th vs
(K+1)-th gap at some scored level is below 1e-3 (at most 0.1% of the queries); the variant
leaf scores of the selected leaves within 1e-4 + 1e-5 |u|; decode selections per step.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W
from oracle import pisa as oracle

import gpu_harness as H

pytestmark = pytest.mark.gpu


def leaf_score(qg: np.ndarray, keys: np.ndarray, j: int, t: int, score: str) -> float:
    """Oracle leaf score of block j for token t: the variant over its keys <= t, summed over heads."""
    blk = keys[j * 64:min((j + 1) * 64, t + 1)]
    z = qg @ blk.T / math.sqrt(keys.shape[1])
    return float(oracle.child_score(z, np.ones(z.shape, dtype=bool), score).sum())


def check_variant(w: W.Workload, score: str, label: str, sample: int | None = None, counts: list | None = None):
    """counts: a list that receives (mismatches, queries) instead of this call checking the budget."""
    B, N, G, K = w.batch, w.seq_len, w.group, w.top_k
    H.log(f"[{label}] inputs B={B} N={N} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} K={K} score={score}")
    q, k, _ = W.prefill_inputs(w, bits=True)
    qd, kd = H.to_device(q, w), H.to_device(k, w)
    pyr = binding.build_pyramid(kd)
    sel, sel_u = binding.select_blocks(qd, kd, pyr, K, return_scores=True, score=score)
    torch.cuda.synchronize()
    sel, sel_u = sel.cpu().numpy(), sel_u.cpu().numpy()
    n_bad = n_total = 0
    max_du = 0.0
    for b in range(B):
        for kvh in range(w.n_kv_heads):
            ts = np.arange(N) if sample is None else H.sample_tokens(N, sample, 17 + b + kvh)
            qg = H.host_values(q[b, :, kvh * G:(kvh + 1) * G]).astype(np.float64)
            kk = H.host_values(k[b, :, kvh]).astype(np.float64)
            opyr = oracle.build_pyramid(kk)
            osel = np.zeros((len(ts), K), dtype=np.int64)
            ogap = np.zeros(len(ts))
            for s in range(0, len(ts), 64):
                tc = ts[s:s + 64]
                osel[s:s + 64], ogap[s:s + 64] = oracle.route(qg[tc], kk, opyr, tc, K, score=score)
            nb, agree = H.compare_selection(sel[b, kvh, ts], osel, ogap, label)
            n_bad += nb
            n_total += len(ts)
            for r in np.nonzero(agree)[0][:: max(1, len(ts) // 200)]:
                t = int(ts[r])
                for slot, j in enumerate(osel[r]):
                    if j < 0:
                        continue
                    want = leaf_score(qg[t], kk, int(j), t, score)
                    du = abs(float(sel_u[b, kvh, t, slot]) - want)
                    max_du = max(max_du, du)
                    assert du <= 1e-4 + 1e-5 * abs(want), (label, t, j, float(sel_u[b, kvh, t, slot]), want)
    if counts is None:
        H.assert_mismatch_budget(n_bad, n_total, label)
    else:
        counts.append((n_bad, n_total))
    H.log(f"[{label}] max |du| on selected leaves {max_du:.3g}")


@pytest.mark.parametrize("score", ["mean", "mean_var"])
@pytest.mark.parametrize("name", ["tiny_f32_n1024", "prefill_n4096"])
def test_variant_prefill_full(name, score):
    check_variant(W.WORKLOADS[name], score, f"{name}_{score}")


@pytest.mark.parametrize("score", ["mean", "mean_var"])
def test_variant_ragged_multi_head(score):
    w = W.WORKLOADS["prefill_n4096"].with_(name="ragged", batch=2, seq_len=4133, n_q_heads=8, n_kv_heads=2,
                                           top_k=6, seed=71)
    check_variant(w, score, f"ragged_{score}", sample=800)


@pytest.mark.parametrize("score", ["mean", "mean_var"])
def test_variant_full_size_sampled(score):
    check_variant(W.WORKLOADS["prefill_n262144"], score, f"prefill_n262144_{score}", sample=400)


@pytest.mark.parametrize("score", ["mean", "mean_var"])
def test_variant_decode(score):
    """Decode with the variant score across leaf and level boundaries (ctx 1000 -> 1130, G = 4, K = 4)."""
    w = W.WORKLOADS["decode_b64_ctx131072"].with_(name="dec_var", batch=1, n_q_heads=8, n_kv_heads=2, top_k=4,
                                                  seed=81)
    n0, steps, G, K, d = 1000, 130, w.group, w.top_k, w.head_dim
    cap = n0 + steps
    _, k0, v0 = W.prefill_inputs(w.with_(seq_len=n0), batches=[0], bits=True, with_q=False)
    kc = torch.zeros((1, cap, w.n_kv_heads, d), dtype=torch.bfloat16, device=H.DEV)
    vc = torch.zeros_like(kc)
    kc[:, :n0] = H.to_device(k0, w)
    vc[:, :n0] = H.to_device(v0, w)
    pyr = binding.build_pyramid(kc, n=n0, capacity=cap)
    toks = {name: np.stack([W.decode_tokens(w, name, 0, h) for h in range(nh)], axis=1)[None]
            for name, nh in (("q", w.n_q_heads), ("k", w.n_kv_heads), ("v", w.n_kv_heads))}
    dq, dk, dv = (H.to_device(toks[x][:, :steps], w) for x in ("q", "k", "v"))
    sels = []
    for s in range(steps):
        _, sel = binding.decode_step(dq[:, s].contiguous(), dk[:, s].contiguous(), dv[:, s].contiguous(),
                                     kc, vc, pyr, n0 + s, K, out_dtype=torch.float32, score=score)
        sels.append(sel.cpu().numpy())
    n_bad = n_total = 0
    for kvh in range(w.n_kv_heads):
        st = oracle.DecodeState(H.host_values(k0[0, :, kvh]).astype(np.float64),
                                H.host_values(v0[0, :, kvh]).astype(np.float64), capacity=cap)
        for s in range(steps):
            qh = H.host_values(toks["q"][0, s, kvh * G:(kvh + 1) * G]).astype(np.float64)
            kn = H.host_values(toks["k"][0, s, kvh]).astype(np.float64)
            vn = H.host_values(toks["v"][0, s, kvh]).astype(np.float64)
            osel, ogap, _, _ = st.step(qh, kn, vn, K, score=score)
            n_total += 1
            if not np.array_equal(sels[s][0, kvh], osel):
                assert ogap < H.GAP_LIMIT, (score, kvh, s, sels[s][0, kvh].tolist(), osel.tolist(), ogap)
                n_bad += 1
    H.assert_mismatch_budget(n_bad, n_total, f"decode_{score}")
