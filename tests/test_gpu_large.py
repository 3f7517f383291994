"""GPU parity at the largest lengths the path is sized for, on the 256K recipe (16 query heads on one
KV head, d = 128, K = 16) drawn on the device with torch's seeded generator
(workloads.device_prefill_inputs); the oracle reads host copies of the same bf16 values.

* N = 999999, the longest selection (up to 10^6 tokens; 15625 leaf blocks, the last one 63 keys):
  pyramid, selection and attention, whose passes run in the sorted token order.  2000 sampled
  tokens, edges and leaf boundaries included: selections by the boundary rule (0.1% budget), leaf
  scores of the selected leaves, the end-to-end attention rows, and the attention on the oracle's
  own selection.
* N = 1048613 (16385 leaf blocks, one more than the token-order kernels take, the last one 37 keys):
  the selection refuses the length, and the attention, given a seeded random selection, keeps
  position order; sampled rows against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_harness as H
from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W
from oracle import pisa as oracle
from test_gpu_order import layout

pytestmark = pytest.mark.gpu

SAMPLE = 2000


def host(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def test_prefill_max_length_sampled():
    n = 999999
    w = W.WORKLOADS["prefill_n262144"].with_(name=f"max_{n}", seq_len=n)
    G, K, d = w.group, w.top_k, w.head_dim
    label = f"max_n{n}"
    H.log(f"[{label}] device-drawn inputs B=1 N={n} Hq={w.n_q_heads} Hkv=1 d={d} K={K}")
    q, k, v = W.device_prefill_inputs(w, n, seed=5, with_v=True)
    pyr = binding.build_pyramid(k)
    sel, sel_u = binding.select_blocks(q, k, pyr, K, return_scores=True)
    cfg = binding.make_cfg(1, n, w.n_q_heads, 1, d, K, q.dtype)
    lay = layout(1, n, w.n_q_heads, 1, d)
    assert binding.attn_workspace_bytes(cfg) == lay["total"]
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=H.DEV)
    o = binding.sparse_attn_fwd(q, k, v, sel, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    stats = ws[lay["stats"]:lay["stats"] + 16].cpu().numpy().view(np.uint64)
    H.log(f"[{label}] adjacent-token share {int(stats[1])} of {int(stats[0])} entries")
    assert stats[0] > 0 and 4 * int(stats[1]) < int(stats[0])          # the sorted order ran

    ts = H.sample_tokens(n, SAMPLE, seed=17)
    ts_d = torch.from_numpy(ts).to(H.DEV)
    kk, vv = host(k[0, :, 0]), host(v[0, :, 0])
    qs = host(q[0, ts_d])                                  # [T, G, d]
    H.log(f"[{label}] oracle on {len(ts)} tokens")
    pyr_o = oracle.build_pyramid(kk)
    sels, gaps = [], []
    for s in range(0, len(ts), 64):
        so, go = oracle.route(qs[s:s + 64], kk, pyr_o, ts[s:s + 64], K)
        sels.append(so)
        gaps.append(go)
    osel, gap = np.concatenate(sels), np.concatenate(gaps)
    gsel = sel[0, 0, ts_d].cpu().numpy()
    n_bad, agree = H.compare_selection(gsel, osel, gap, label)
    H.assert_mismatch_budget(n_bad, len(ts), label)

    # leaf scores of the selected leaves, on every 10th agreeing row
    gu = sel_u[0, 0, ts_d].cpu().numpy()
    for r in np.nonzero(agree)[0][::10]:
        for slot, j in enumerate(osel[r]):
            if j >= 0:
                want = float(np.sum(oracle.leaf_lse(qs[r], kk, int(j), int(ts[r]))))
                assert abs(float(gu[r, slot]) - want) <= 1e-4 + 1e-5 * abs(want), (label, int(ts[r]), int(j))

    tol_abs, tol_rel = H.attn_tolerance(w)
    want_o, want_lse, _ = oracle.attention(qs, kk, vv, osel, ts)
    got = o[0, ts_d].cpu().numpy()
    ma, rl = H.attn_errors(got[agree], want_o[agree])
    H.log(f"[{label}] end-to-end attention max-abs {ma:.3g} rel-L2 {rl:.3g}")
    assert ma <= tol_abs and rl <= tol_rel, (label, ma, rl)

    # the attention on the oracle's own selection, every sampled row
    sel_in = sel.clone()
    sel_in[0, 0, ts_d] = torch.from_numpy(osel.astype(np.int32)).to(H.DEV)
    o2, lse2 = binding.sparse_attn_fwd(q, k, v, sel_in, return_lse=True, out_dtype=torch.float32)
    ma, rl = H.attn_errors(o2[0, ts_d].cpu().numpy(), want_o)
    H.log(f"[{label}] attention on the oracle selection max-abs {ma:.3g} rel-L2 {rl:.3g}")
    assert ma <= tol_abs and rl <= tol_rel, (label, ma, rl)
    np.testing.assert_allclose(lse2[0, :, ts_d].cpu().numpy().T, want_lse, atol=2e-4)


def test_attention_past_the_order_limit_sampled():
    n = 1048576 + 37
    w = W.WORKLOADS["prefill_n262144"].with_(name=f"max_{n}", seq_len=n)
    K, d = w.top_k, w.head_dim
    label = f"attn_n{n}"
    H.log(f"[{label}] device-drawn inputs B=1 N={n} Hq={w.n_q_heads} Hkv=1 d={d} K={K}")
    q, k, v = W.device_prefill_inputs(w, n, seed=6, with_v=True)
    pyr = binding.build_pyramid(k)
    with pytest.raises(RuntimeError, match="unsupported configuration"):
        binding.select_blocks(q, k, pyr, K)
    # a seeded random selection: K draws per token from its valid blocks 0 .. t / 64, sorted (a
    # repeated id counts once on both sides)
    rng = np.random.default_rng(19)
    m = (np.arange(n) // 64 + 1)[:, None]
    sel = np.sort(np.floor(rng.random((n, K)) * m).astype(np.int32), axis=1)
    cfg = binding.make_cfg(1, n, w.n_q_heads, 1, d, K, q.dtype)
    assert binding.attn_workspace_bytes(cfg) == lay_no_order(n, w.n_q_heads, d)   # no order arrays
    seld = torch.from_numpy(sel).to(H.DEV).view(1, 1, n, K)
    o, lse = binding.sparse_attn_fwd(q, k, v, seld, return_lse=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ts = H.sample_tokens(n, SAMPLE, seed=23)
    ts_d = torch.from_numpy(ts).to(H.DEV)
    kk, vv = host(k[0, :, 0]), host(v[0, :, 0])
    qs = host(q[0, ts_d])
    H.log(f"[{label}] oracle attention on {len(ts)} tokens")
    want_o, want_lse, _ = oracle.attention(qs, kk, vv, sel[ts], ts)
    ma, rl = H.attn_errors(o[0, ts_d].cpu().numpy(), want_o)
    H.log(f"[{label}] attention max-abs {ma:.3g} rel-L2 {rl:.3g}")
    tol_abs, tol_rel = H.attn_tolerance(w)
    assert ma <= tol_abs and rl <= tol_rel, (label, ma, rl)
    np.testing.assert_allclose(lse[0, :, ts_d].cpu().numpy().T, want_lse, atol=2e-4)


def lay_no_order(n: int, hq: int, d: int) -> int:
    """Attention workspace bytes past 16384 leaf blocks: packed K and V, then the (m, l) pairs."""
    up = lambda x: -(-x // 256) * 256
    m1 = -(-n // 64)
    return 2 * up(m1 * 64 * d * 2) + up(hq * n * 8)
