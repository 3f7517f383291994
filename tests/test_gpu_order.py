"""The token order of the attention passes (order.hip), read back from the attention workspace and
checked against a plain host computation of the same rule:

* the adjacent-token statistic: over every 64th token t (t = 1, 65, ...), the valid entries of row t
  and how many of them row t - 1 also lists among its valid entries;
* the choice: sorted order when fewer than a quarter of those entries are shared;
* with the sorted order, for each pass p (two for a float32 output, one for bfloat16): every token's
  key is its smallest valid block j with j % passes == p that was selected at most 4 * 64 * K times
  in the whole call (else ceil(N / 64)), and the pass's order is the tokens sorted by key with ties
  in position order;
* the attention output is the same bit for bit whichever order runs (the natural order is forced
  by a selection whose rows repeat the previous row's blocks), and matches the oracle.

Memory layout of the workspace (the library's attention workspace, 256-byte aligned arrays): packed
K and V blocks, the per-head (m, l) pairs, block counts, key counts per chunk of 4096 tokens, key
totals, two uint64 statistics, keys, order.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_harness as H
from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W
from oracle import pisa as oracle

pytestmark = pytest.mark.gpu

SAMPLE = 64
PASSES = 2


def up(x: int) -> int:
    return -(-x // 256) * 256


def layout(B, N, Hq, Hkv, d):
    m1 = -(-N // 64)
    bh = B * Hkv
    pack = up(bh * m1 * 64 * d * 2)
    hist = 2 * pack + up(B * Hq * N * 8)
    keycnt = hist + up(bh * m1 * 4)
    chunks = -(-N // 4096)                                    # the sort's chunks of 4096 tokens
    keytot = keycnt + up(PASSES * bh * (m1 + 1) * chunks * 4)
    stats = keytot + up(PASSES * bh * (m1 + 1) * 4)
    keys = stats + 256
    order = keys + up(PASSES * bh * N * 4)
    total = order + up(PASSES * bh * N * 4)
    return dict(m1=m1, bh=bh, hist=hist, stats=stats, keys=keys, order=order, total=total)


def host_rule(sel: np.ndarray, K: int, passes: int = PASSES):
    """sel [bh, N, K] -> (entries, overlap, sorted?, keys [passes, bh, N])."""
    bh, N, _ = sel.shape
    m1 = -(-N // 64)
    t = np.arange(N)[None, :, None]
    valid = (sel >= 0) & (sel <= t // 64)
    entries = overlap = 0
    for b in range(bh):
        for tt in range(1, N, SAMPLE):
            prev = set(int(j) for j, ok in zip(sel[b, tt - 1], valid[b, tt - 1]) if ok)
            for j, ok in zip(sel[b, tt], valid[b, tt]):
                if ok:
                    entries += 1
                    overlap += int(j) in prev
    is_sorted = entries > 0 and overlap * 4 < entries
    hist = np.zeros((bh, m1), np.int64)
    for b in range(bh):
        np.add.at(hist[b], sel[b][valid[b]], 1)
    keys = np.full((passes, bh, N), m1, np.int64)
    for b in range(bh):
        cold = valid[b] & (hist[b][np.clip(sel[b], 0, m1 - 1)] <= 4 * 64 * K)
        for p in range(passes):
            keys[p, b] = np.where(cold & (sel[b] % passes == p), sel[b], m1).min(-1)
    return entries, overlap, is_sorted, keys


def run(w: W.Workload, sel: np.ndarray, out_dtype=torch.float32):
    q, k, v = W.prefill_inputs(w, bits=True)
    qd, kd, vd = H.to_device(q, w), H.to_device(k, w), H.to_device(v, w)
    B, N, Hq, d = qd.shape
    lay = layout(B, N, Hq, w.n_kv_heads, d)
    cfg = binding.make_cfg(B, N, Hq, w.n_kv_heads, d, w.top_k, qd.dtype)
    assert binding.attn_workspace_bytes(cfg) == lay["total"]
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device=H.DEV)
    seld = torch.from_numpy(sel.astype(np.int32).reshape(B, w.n_kv_heads, N, w.top_k)).to(H.DEV)
    o = binding.sparse_attn_fwd(qd, kd, vd, seld, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    stats = raw[lay["stats"]:lay["stats"] + 16].view(np.uint64)
    bhN = lay["bh"] * N
    keys = raw[lay["keys"]:lay["keys"] + PASSES * bhN * 4].view(np.int32).reshape(PASSES, lay["bh"], N)
    order = raw[lay["order"]:lay["order"] + PASSES * bhN * 4].view(np.int32).reshape(PASSES, lay["bh"], N)
    return (q, k, v), o.float().cpu().numpy(), stats, keys, order


def check_case(w: W.Workload, sel: np.ndarray, want_sorted: bool, label: str, out_dtype=torch.float32):
    """A float32 output runs two passes (even, then odd block ids), a bfloat16 output one."""
    bh = w.batch * w.n_kv_heads
    passes = PASSES if out_dtype == torch.float32 else 1
    sel3 = sel.reshape(bh, w.seq_len, w.top_k)
    entries, overlap, is_sorted, keys_want = host_rule(sel3, w.top_k, passes)
    assert is_sorted == want_sorted, (label, entries, overlap)
    (q, k, v), o, stats, keys, order = run(w, sel, out_dtype)
    H.log(f"[{label}] entries {int(stats[0])} overlap {int(stats[1])} (host {entries} / {overlap}), "
          f"{'sorted' if is_sorted else 'natural'} order")
    assert int(stats[0]) == entries and int(stats[1]) == overlap, (label, stats, entries, overlap)
    if is_sorted:
        np.testing.assert_array_equal(keys[:passes], keys_want)
        for p in range(passes):
            for b in range(bh):
                want = np.lexsort((np.arange(w.seq_len), keys_want[p, b]))
                np.testing.assert_array_equal(order[p, b], want, err_msg=f"{label} pass {p} unit {b}")
    # the output against the oracle on the same rows, every token
    G = w.group
    tol_abs, tol_rel = H.attn_tolerance(w)
    for b in range(w.batch):
        for kvh in range(w.n_kv_heads):
            want, _, _ = oracle.attention(H.host_values(q[b][:, kvh * G:(kvh + 1) * G]).astype(np.float64),
                                          H.host_values(k[b, :, kvh]).astype(np.float64),
                                          H.host_values(v[b, :, kvh]).astype(np.float64),
                                          sel[b, kvh], np.arange(w.seq_len))
            got = o[b][:, kvh * G:(kvh + 1) * G]
            if out_dtype == torch.float32:
                ma, rl = H.attn_errors(got, want)
                assert ma <= tol_abs and rl <= tol_rel, (label, b, kvh, ma, rl)
            else:
                H.assert_bf16_output(got, want, label)
    return o


def test_order_statistics_keys_and_permutation():
    """Random rows (little sharing: sorted order) and rows that repeat the previous token's blocks
    (natural order), on the same inputs: statistics, keys and orders as the host computes them, and
    both outputs within the tolerance of the oracle; the rows of the shared blocks agree bit for bit
    between the two calls where both list the same blocks."""
    # 188 leaf blocks: random rows of 6 share about 3% of their blocks with the previous row
    w = W.WORKLOADS["prefill_n4096"].with_(name="order", seq_len=12000, batch=1, n_q_heads=8, n_kv_heads=2,
                                           top_k=6, seed=61)
    rng = np.random.default_rng(62)
    N, K = w.seq_len, w.top_k
    rand = np.full((w.batch, w.n_kv_heads, N, K), -1, np.int64)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            for t in range(N):
                m = t // 64 + 1
                rand[b, h, t, :min(K, m)] = np.sort(rng.choice(m, size=min(K, m), replace=False))
    o_sorted = check_case(w, rand, True, "random rows")
    # each row: the previous row's blocks, the oldest one swapped for the newest valid block
    rep = rand.copy()
    for t in range(1, N):
        prev = rep[:, :, t - 1]
        new = np.concatenate([prev[..., 1:], np.full(prev.shape[:-1] + (1,), t // 64)], axis=-1)
        rep[:, :, t] = np.where((prev >= 0).all(-1, keepdims=True), new, rand[:, :, t])
    o_natural = check_case(w, rep, False, "repeated rows")
    # one pass (bfloat16 output): the keys and the order of the single pass
    check_case(w, rand, True, "random rows, one pass", out_dtype=torch.bfloat16)
    # tokens whose rows are equal in both selections: the same output bits in either order
    same = np.all(rand == rep, axis=-1)                       # [B, Hkv, N]
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            rows = same[b, h]
            cols = slice(h * w.group, (h + 1) * w.group)
            assert np.array_equal(o_sorted[b, rows][:, cols], o_natural[b, rows][:, cols])
