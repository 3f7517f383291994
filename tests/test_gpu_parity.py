"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs.  See tests/gpu_harness.py for the comparison rules."""
import numpy as np
import pytest
import torch

from hierarchical_top_selection_amd import binding
from hierarchical_top_selection_amd import workloads as W
from oracle import pisa as oracle

import gpu_harness as H

pytestmark = pytest.mark.gpu


def _pyramid_levels(flat: np.ndarray, n: int, capacity: int):
    """Split a capacity-layout pyramid [nodes, d] into the levels of length n."""
    cap_sizes = oracle.level_sizes(capacity)
    sizes = oracle.level_sizes(n)
    out, off = [], 0
    for lvl, cap in enumerate(cap_sizes):
        if lvl < len(sizes):
            out.append(flat[off:off + sizes[lvl]])
        off += cap
    return out


def check_prefill(w: W.Workload, label: str, sample: int | None = None, seed: int = 0, inputs=None,
                  attn_abs: float | None = None, counts: list | None = None):
    """inputs: (q, k, v) storage arrays to use instead of the workload's own draw; attn_abs: a
    max-abs gate for the attention outputs in place of the workload's; counts: a list that
    receives (mismatches, queries) instead of this call checking the budget on its own."""
    B, N, G, K = w.batch, w.seq_len, w.group, w.top_k
    H.log(f"[{label}] inputs B={B} N={N} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} K={K} {w.dtype}")
    q, k, v = W.prefill_inputs(w, bits=True) if inputs is None else inputs
    H.log(f"[{label}] GPU pyramid + select + attention")
    g = H.run_gpu_prefill(w, q, k, v)
    pyr = g["pyr"].cpu().numpy()
    sel = g["sel"].cpu().numpy()
    sel_u = g["sel_u"].cpu().numpy()
    o = g["o"].cpu().numpy()
    o_native = g["o_native"].float().cpu().numpy()
    sel_in = g["sel"].clone()
    n_bad = n_total = 0
    units = []
    max_du = 0.0
    for b in range(B):
        for kvh in range(w.n_kv_heads):
            ts = np.arange(N) if sample is None else H.sample_tokens(N, sample, seed + 7 * b + kvh)
            H.log(f"[{label}] oracle b={b} kvh={kvh} on {len(ts)} tokens")
            ora = H.oracle_prefill(w, q, k, v, b, kvh, ts)
            # pyramid: fp32 sums in key order vs the fp64 mean
            kk = H.host_values(k[b, :, kvh]).astype(np.float64)
            for got, want in zip(_pyramid_levels(pyr[b, kvh], N, N), oracle.build_pyramid(kk)):
                np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-5)
            nb, agree = H.compare_selection(sel[b, kvh, ts], ora["sel"], ora["gap"], label)
            n_bad += nb
            n_total += len(ts)
            # exact leaf scores of the selected leaves (rows that agree)
            qg = H.host_values(q[b, :, kvh * G:(kvh + 1) * G]).astype(np.float64)
            for r in np.nonzero(agree)[0][:: max(1, len(ts) // 200)]:
                t = int(ts[r])
                for slot, j in enumerate(ora["sel"][r]):
                    if j < 0:
                        continue
                    want = float(np.sum(oracle.leaf_lse(qg[t], kk, int(j), t)))
                    du = abs(float(sel_u[b, kvh, t, slot]) - want)
                    max_du = max(max_du, du)
                    assert du <= 1e-4 + 1e-5 * abs(want), (label, t, j, sel_u[b, kvh, t, slot], want)
            # end-to-end attention where the selections agree
            heads = slice(kvh * G, (kvh + 1) * G)
            tol_abs, tol_rel = H.attn_tolerance(w)
            tol_abs = tol_abs if attn_abs is None else attn_abs
            ma, rl = H.attn_errors(o[b, ts][:, heads][agree], ora["o"][agree])
            assert ma <= tol_abs and rl <= tol_rel, (label, "end-to-end", ma, rl)
            if w.dtype == "bf16":
                H.assert_bf16_output(o_native[b, ts][:, heads][agree], ora["o"][agree], label, abs_gate=tol_abs)
            sel_in[b, kvh, torch.from_numpy(ts).to(H.DEV)] = torch.from_numpy(ora["sel"].astype(np.int32)).to(H.DEV)
            units.append((b, kvh, ts, ora))
    if counts is None:
        H.assert_mismatch_budget(n_bad, n_total, label)
    else:
        counts.append((n_bad, n_total))
    H.log(f"[{label}] max |du| on selected leaves {max_du:.3g}")
    # attention on the oracle's own selection (fed to the kernel as input)
    o2, lse2 = binding.sparse_attn_fwd(g["q"], g["k"], g["v"], sel_in, return_lse=True, out_dtype=torch.float32)
    o2 = o2.cpu().numpy()
    lse2 = lse2.cpu().numpy()
    worst = (0.0, 0.0)
    for b, kvh, ts, ora in units:
        heads = slice(kvh * G, (kvh + 1) * G)
        ma, rl = H.attn_errors(o2[b, ts][:, heads], ora["o"])
        worst = (max(worst[0], ma), max(worst[1], rl))
        tol_abs, tol_rel = H.attn_tolerance(w)
        tol_abs = tol_abs if attn_abs is None else attn_abs
        assert ma <= tol_abs and rl <= tol_rel, (label, b, kvh, ma, rl)
        np.testing.assert_allclose(lse2[b, heads][:, ts].T, ora["lse"], atol=2e-4 if w.dtype == "bf16" else 2e-5)
    H.log(f"[{label}] attention on oracle selection: max-abs {worst[0]:.3g} rel-L2 {worst[1]:.3g}")
    return g


@pytest.mark.parametrize("name", ["tiny_f32_n1024", "prefill_n4096"])
def test_prefill_full(name):
    check_prefill(W.WORKLOADS[name], name)


def test_prefill_ragged_multi_head():
    w = W.WORKLOADS["prefill_n4096"].with_(name="ragged", batch=2, seq_len=4133, n_q_heads=32, n_kv_heads=2,
                                           top_k=8, seed=11)
    check_prefill(w, "ragged_b2_n4133_k8", sample=1500)


@pytest.mark.parametrize("d,hq,hkv,K,n,dtype", [
    (64, 8, 1, 6, 3000, "bf16"),      # d = 64, G = 8
    (128, 2, 2, 5, 2000, "bf16"),     # G = 1
    (128, 4, 2, 3, 1500, "bf16"),     # G = 2
    (64, 16, 1, 2, 1100, "f32"),      # fp32, G = 16, small K
    (128, 4, 1, 32, 2600, "bf16"),    # K = 32 > number of leaves / 2
])
def test_prefill_shapes(d, hq, hkv, K, n, dtype):
    w = W.WORKLOADS["prefill_n4096"].with_(name="shape", head_dim=d, n_q_heads=hq, n_kv_heads=hkv, top_k=K,
                                           seq_len=n, dtype=dtype, seed=20 + d + hq + K)
    check_prefill(w, f"shape_d{d}_g{hq // hkv}_k{K}_n{n}_{dtype}")


@pytest.mark.parametrize("n", [1, 50, 64, 65, 130, 257])
def test_prefill_tiny_lengths(n):
    w = W.WORKLOADS["prefill_n4096"].with_(name="short", seq_len=n, top_k=2, n_q_heads=4, seed=30 + n)
    check_prefill(w, f"short_n{n}")


def _leaf_sums_log2(q: np.ndarray, k: np.ndarray, G: int, scale: float) -> np.ndarray:
    """log2 of sum_k 2^(q_h . k c2) over each causal leaf of each token's first KV head (fp64), for
    every head: [N, M1, G]; -inf where the leaf starts after the token."""
    N = q.shape[1]
    m1 = -(-N // 64)
    qq = H.host_values(q[0, :, :G]).astype(np.float64)            # [N, G, d]
    kk = H.host_values(k[0, :, 0]).astype(np.float64)             # [N, d]
    y = np.einsum("tgd,sd->tgs", qq, kk) * scale * np.log2(np.e)  # [N, G, N]
    y = np.where(np.arange(N)[None, None, :] <= np.arange(N)[:, None, None], y, -np.inf)
    out = np.full((N, m1, G), -np.inf)
    for j in range(m1):
        blk = y[:, :, 64 * j:64 * j + 64]
        m = blk.max(-1)
        with np.errstate(invalid="ignore"):
            out[:, j] = m + np.log2(np.exp2(blk - m[..., None]).sum(-1))
    return out


@pytest.mark.parametrize("regime", ["wide", "large", "negative"])
def test_prefill_logit_ranges(regime):
    """Stage 2 sums 2^(scaled logit) with no shift while every head's sum lies in [2^-60, 2^60] and
    takes the max-shifted sum otherwise.  Inputs whose leaf sums fall on both sides of that range
    ("wide": queries and keys scaled by 4), above it everywhere ("large": by 8) and below it
    ("negative": keys along +u, queries along -u, so every logit is far below zero) must still match
    the oracle: selections by the boundary rule, leaf scores and outputs.

    With logits this far apart a row's softmax sits on one or two keys, so the rounding of P to
    bf16 before the P V product (at most 2^-8 of each weight) no longer averages out: the output
    can be off by up to 2^-8 max |v|, which is the max-abs gate here (plus 1e-3 for the fp32 sums);
    the relative-L2 gate is the workload's."""
    w = W.WORKLOADS["prefill_n4096"].with_(name=f"range_{regime}", seq_len=1500, batch=1, n_q_heads=8,
                                           n_kv_heads=1, top_k=4, seed=41)
    q, k, v = W.prefill_inputs(w)                                  # float32 values
    d = w.head_dim
    if regime == "wide":
        q, k = q * 4.0, k * 4.0
    elif regime == "large":
        q, k = q * 8.0, k * 8.0
    else:
        u = np.random.default_rng(42).standard_normal(d)
        u /= np.linalg.norm(u)
        q = q - 40.0 * u
        k = k + 40.0 * u
    q, k, v = (W.to_storage(x.astype(np.float32), "bf16") for x in (q, k, v))
    s2 = _leaf_sums_log2(q, k, w.group, 1.0 / np.sqrt(d))
    causal = np.isfinite(s2)
    outside = causal & ((s2 < -60) | (s2 > 60))
    frac = outside.sum() / causal.sum()
    H.log(f"[range {regime}] {frac:.3f} of (token, leaf, head) sums outside [2^-60, 2^60]")
    if regime == "wide":
        assert 0.01 < frac < 0.99
    else:
        assert frac > 0.99
    vmax = float(np.abs(H.host_values(v)).max())
    check_prefill(w, f"range_{regime}", inputs=(q, k, v), attn_abs=vmax / 256.0 + 1e-3)


def test_all_leaves_selected_is_dense_causal_attention():
    w = W.WORKLOADS["prefill_n4096"].with_(name="dense", seq_len=700, top_k=12, seed=41)
    q, k, v = W.prefill_inputs(w, bits=True)
    g = H.run_gpu_prefill(w, q, k, v)
    sel = g["sel"].cpu().numpy()[0, 0]
    for t in range(700):
        assert [x for x in sel[t] if x >= 0] == list(range(t // 64 + 1))
    ts = np.arange(0, 700, 7)
    want = oracle.dense_causal_attention(H.host_values(q[0]).astype(np.float64)[ts],
                                         H.host_values(k[0, :, 0]).astype(np.float64),
                                         H.host_values(v[0, :, 0]).astype(np.float64), ts)
    ma, rl = H.attn_errors(g["o"].cpu().numpy()[0, ts], want)
    assert ma <= 1e-2 and rl <= 5e-3, (ma, rl)


def test_strided_inputs_match_contiguous():
    """Q/K/V as views into one packed [B, N, Hq + 2 Hkv, d] buffer give identical results."""
    w = W.WORKLOADS["prefill_n4096"].with_(name="strided", seq_len=2000, batch=2, n_q_heads=8, n_kv_heads=2,
                                           top_k=4, seed=43)
    q, k, v = W.prefill_inputs(w, bits=True)
    ref = H.run_gpu_prefill(w, q, k, v)
    packed = torch.cat([H.to_device(q, w), H.to_device(k, w), H.to_device(v, w)], dim=2)
    qs, ks, vs = packed[:, :, :8], packed[:, :, 8:10], packed[:, :, 10:12]
    assert not qs.is_contiguous()
    pyr = binding.build_pyramid(ks)
    sel = binding.select_blocks(qs, ks, pyr, 4)
    o = binding.sparse_attn_fwd(qs, ks, vs, sel)
    assert torch.equal(pyr, ref["pyr"]) and torch.equal(sel, ref["sel"]) and torch.equal(o, ref["o_native"])


def _parity_selection(n: int, K: int, seed: int) -> np.ndarray:
    """Selection rows that stress the even / odd block-id passes of the float32-output attention:
    by t % 5, only even blocks, only odd blocks, no block at all, valid blocks with -1 holes
    between them, and distinct blocks in random order."""
    rng = np.random.default_rng(seed)
    sel = np.full((n, K), -1, dtype=np.int32)
    for t in range(n):
        valid = np.arange(t // 64 + 1)
        kind = t % 5
        if kind == 0:
            pick = valid[valid % 2 == 0][-K:]
        elif kind == 1:
            pick = valid[valid % 2 == 1][-K:]
        elif kind == 2:
            pick = valid[:0]
        else:
            pick = rng.choice(valid, size=min(len(valid), K // 2 if kind == 3 else K), replace=False)
            if kind == 3:
                pick = np.sort(pick)
        if kind == 3:
            sel[t, 1:2 * len(pick):2] = pick                 # holes at every even slot
        else:
            sel[t, :len(pick)] = pick
    return sel


def test_attention_block_parities():
    """The float32-output attention (even block ids, then odd ones, the state carried between
    them) and the single-pass bfloat16-output attention against the oracle on selections that
    put every block in one pass, in none, or leave holes."""
    w = W.WORKLOADS["prefill_n4096"].with_(name="parities", seq_len=1800, n_q_heads=8, top_k=8, seed=47)
    q, k, v = W.prefill_inputs(w, bits=True)
    sel = _parity_selection(w.seq_len, w.top_k, seed=48)
    qd, kd, vd = H.to_device(q, w), H.to_device(k, w), H.to_device(v, w)
    seld = torch.from_numpy(sel[None, None]).to(H.DEV)
    o, lse = binding.sparse_attn_fwd(qd, kd, vd, seld, return_lse=True, out_dtype=torch.float32)
    o16 = binding.sparse_attn_fwd(qd, kd, vd, seld)
    torch.cuda.synchronize()
    o, lse, o16 = o.cpu().numpy()[0], lse.cpu().numpy()[0], o16.float().cpu().numpy()[0]
    ts = np.arange(w.seq_len)
    with np.errstate(invalid="ignore"):                 # rows without a block: -inf - (-inf), not compared
        want, want_lse, _ = oracle.attention(H.host_values(q[0]).astype(np.float64),
                                             H.host_values(k[0, :, 0]).astype(np.float64),
                                             H.host_values(v[0, :, 0]).astype(np.float64), sel, ts)
    empty = np.all(sel < 0, axis=1)
    assert empty.sum() > 0 and np.all(o[empty] == 0.0) and np.all(o16[empty] == 0.0)
    assert np.all(np.isneginf(lse[:, empty]))
    ma, rl = H.attn_errors(o[~empty], want[~empty])
    assert ma <= 1e-2 and rl <= 5e-3, (ma, rl)
    H.assert_bf16_output(o16[~empty], want[~empty], "parities bf16")
    np.testing.assert_allclose(lse[:, ~empty].T, want_lse[~empty], atol=2e-4)
    H.log(f"[parities] max-abs {ma:.3g} rel-L2 {rl:.3g} over {int((~empty).sum())} rows, {int(empty.sum())} empty")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_ignores_negative_future_and_repeated_ids(dtype):
    """Selection rows with -1, repeated ids, ids past t, past the last block, INT32_MAX and INT32_MIN:
    every path (two-pass float32 output, one-pass bfloat16 output, float32 inputs) attends over the
    union of the listed blocks cut to positions <= t, as the oracle does on the same rows."""
    w = W.WORKLOADS["prefill_n4096"].with_(name="bad_ids", seq_len=1300, n_q_heads=8, top_k=12, seed=49,
                                           dtype=dtype)
    N, K = w.seq_len, w.top_k
    m1 = -(-N // 64)
    rng = np.random.default_rng(50)
    sel = np.full((N, K), -1, dtype=np.int64)
    for t in range(N):
        valid = np.arange(t // 64 + 1)
        pick = list(rng.choice(valid, size=min(len(valid), 4), replace=False))
        row = pick + pick[:2] + [t // 64 + 1, m1, m1 + 7, 2 ** 31 - 1, -2 ** 31, -1]
        sel[t, :len(row)] = rng.permutation(row)[:K]
    q, k, v = W.prefill_inputs(w, bits=True)
    qd, kd, vd = H.to_device(q, w), H.to_device(k, w), H.to_device(v, w)
    seld = torch.from_numpy(sel.astype(np.int32)[None, None]).to(H.DEV)
    H.log(f"[bad_ids {dtype}] GPU attention")
    o, lse = binding.sparse_attn_fwd(qd, kd, vd, seld, return_lse=True, out_dtype=torch.float32)
    o_native = binding.sparse_attn_fwd(qd, kd, vd, seld)
    torch.cuda.synchronize()
    want, want_lse, _ = oracle.attention(H.host_values(q[0]).astype(np.float64),
                                         H.host_values(k[0, :, 0]).astype(np.float64),
                                         H.host_values(v[0, :, 0]).astype(np.float64), sel, np.arange(N))
    tol_abs, tol_rel = H.attn_tolerance(w)
    ma, rl = H.attn_errors(o.cpu().numpy()[0], want)
    assert ma <= tol_abs and rl <= tol_rel, (dtype, ma, rl)
    np.testing.assert_allclose(lse.cpu().numpy()[0].T, want_lse, atol=2e-4 if dtype == "bf16" else 2e-5)
    if dtype == "bf16":
        H.assert_bf16_output(o_native.float().cpu().numpy()[0], want, "bad_ids bf16 output")
    H.log(f"[bad_ids {dtype}] max-abs {ma:.3g} rel-L2 {rl:.3g}")


def test_repeat_runs_are_bit_identical():
    w = W.WORKLOADS["prefill_n4096"]
    q, k, v = W.prefill_inputs(w, bits=True)
    a = H.run_gpu_prefill(w, q, k, v)
    b = H.run_gpu_prefill(w, q, k, v)
    for key in ("pyr", "sel", "sel_u", "o", "lse", "o_native"):
        assert torch.equal(a[key], b[key]), key


def check_prefill_every_token(w: W.Workload, label: str, pool, chunk: int = 512):
    """Every query token of a full-size workload against the oracle, which runs in the forked pool:
    pyramid, selections under the boundary rule (mismatches pooled over all B * H_kv * N queries),
    leaf scores of the selected leaves, end-to-end attention, and attention on the oracle's own
    selection fed to the kernel."""
    import oracle_pool

    B, N, G, K, Hkv = w.batch, w.seq_len, w.group, w.top_k, w.n_kv_heads
    H.log(f"[{label}] inputs B={B} N={N} Hq={w.n_q_heads} Hkv={Hkv} d={w.head_dim} K={K}; "
          f"oracle on every token in {oracle_pool.worker_count()} processes")
    tasks = [(w, b, kvh, np.arange(s0, min(s0 + chunk, N)), K)
             for b in range(B) for kvh in range(Hkv) for s0 in range(0, N, chunk)]
    pending = pool.imap_unordered(oracle_pool.prefill_chunk, tasks)      # runs while the GPU works
    q, k, v = W.prefill_inputs(w, bits=True)
    H.log(f"[{label}] GPU pyramid + select + attention")
    g = H.run_gpu_prefill(w, q, k, v)
    pyr, sel, sel_u = g["pyr"].cpu().numpy(), g["sel"].cpu().numpy(), g["sel_u"].cpu().numpy()
    o, o_native = g["o"].cpu().numpy(), g["o_native"].float().cpu().numpy()
    ora_sel = np.full((B, Hkv, N, K), -7, dtype=np.int32)
    ora_gap = np.full((B, Hkv, N), np.nan)
    ora_u = np.zeros((B, Hkv, N, K))
    ora_o = np.zeros((B, N, w.n_q_heads, w.head_dim), dtype=np.float32)
    ora_lse = np.zeros((B, w.n_q_heads, N))
    for i, (b, kvh, ts, s_, gp, su, oo, ll) in enumerate(pending):
        ora_sel[b, kvh, ts], ora_gap[b, kvh, ts], ora_u[b, kvh, ts] = s_, gp, su
        ora_o[b, ts, kvh * G:(kvh + 1) * G] = oo
        ora_lse[b, kvh * G:(kvh + 1) * G][:, ts] = ll.T
        if (i + 1) % max(1, len(tasks) // 10) == 0:
            H.log(f"[{label}] oracle {i + 1}/{len(tasks)} chunks")
    assert not np.any(ora_sel == -7) and not np.any(np.isnan(ora_gap))
    for b in range(B):
        for kvh in range(Hkv):
            kk = H.host_values(k[b, :, kvh]).astype(np.float64)
            for got, want in zip(_pyramid_levels(pyr[b, kvh], N, N), oracle.build_pyramid(kk)):
                np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-5)
    # selections: equal sets except at oracle boundary gaps < 1e-3, fewer than 0.1% of all queries
    agree = np.all(sel == ora_sel, axis=-1)
    bad = np.argwhere(~agree)
    for b, kvh, t in bad:
        assert ora_gap[b, kvh, t] < H.GAP_LIMIT, (label, b, kvh, t, sel[b, kvh, t].tolist(),
                                                   ora_sel[b, kvh, t].tolist(), ora_gap[b, kvh, t])
    near = float(np.mean(ora_gap < H.GAP_LIMIT))
    H.log(f"[{label}] {near:.1%} of queries have an oracle gap below 1e-3")
    H.assert_mismatch_budget(len(bad), agree.size, label)
    # leaf scores of the selected leaves where the selections agree
    ok = agree[..., None] & (ora_sel >= 0)
    du = np.abs(sel_u[ok] - ora_u[ok])
    assert np.all(du <= 1e-4 + 1e-5 * np.abs(ora_u[ok])), (label, "leaf scores", float(du.max()))
    assert np.all(np.isneginf(sel_u[agree[..., None] & (ora_sel < 0)]))
    H.log(f"[{label}] max |du| over {int(ok.sum())} selected leaves {du.max():.3g}")
    # end-to-end attention where the selections agree, then on the oracle's selection (every row)
    tol_abs, tol_rel = H.attn_tolerance(w)
    o2, lse2 = binding.sparse_attn_fwd(g["q"], g["k"], g["v"], torch.from_numpy(ora_sel).to(H.DEV),
                                       return_lse=True, out_dtype=torch.float32)
    o2, lse2 = o2.cpu().numpy(), lse2.cpu().numpy()
    worst = [0.0, 0.0, 0.0, 0.0]
    for b in range(B):
        for kvh in range(Hkv):
            heads = slice(kvh * G, (kvh + 1) * G)
            rows = agree[b, kvh]
            ma, rl = H.attn_errors(o[b, rows][:, heads], ora_o[b, rows][:, heads])
            assert ma <= tol_abs and rl <= tol_rel, (label, "end-to-end", b, kvh, ma, rl)
            H.assert_bf16_output(o_native[b, rows][:, heads], ora_o[b, rows][:, heads], label)
            ma2, rl2 = H.attn_errors(o2[b][:, heads], ora_o[b][:, heads])
            assert ma2 <= tol_abs and rl2 <= tol_rel, (label, "oracle selection", b, kvh, ma2, rl2)
            np.testing.assert_allclose(lse2[b, heads], ora_lse[b, heads], atol=2e-4)
            worst = [max(worst[0], ma), max(worst[1], rl), max(worst[2], ma2), max(worst[3], rl2)]
    H.log(f"[{label}] attention end-to-end max-abs {worst[0]:.3g} rel-L2 {worst[1]:.3g}; on the oracle's "
          f"selection max-abs {worst[2]:.3g} rel-L2 {worst[3]:.3g} over {B * N} tokens")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["prefill_n32768", "prefill_n262144"])
def test_prefill_full_size_every_token(name, oracle_workers):
    check_prefill_every_token(W.WORKLOADS[name], name, oracle_workers)


# ----------------------------------------------------------------------------- decode
def run_decode(w: W.Workload, batches, n0: int, steps: int, label: str, check_units=None, counts: list | None = None):
    """counts: a list that receives (mismatches, queries) instead of this call checking the budget."""
    B = len(batches)
    G, K, d = w.group, w.top_k, w.head_dim
    cap = n0 + steps
    H.log(f"[{label}] decode inputs B={B} ctx={n0} steps={steps} Hq={w.n_q_heads} Hkv={w.n_kv_heads} K={K}")
    ctx_w = w.with_(seq_len=n0)
    _, k0, v0 = W.prefill_inputs(ctx_w, batches=batches, bits=True, with_q=False)
    kc = torch.zeros((B, cap, w.n_kv_heads, d), dtype=H.torch_dtype(w), device=H.DEV)
    vc = torch.zeros_like(kc)
    kc[:, :n0] = H.to_device(k0, w)
    vc[:, :n0] = H.to_device(v0, w)
    pyr = binding.build_pyramid(kc, n=n0, capacity=cap)
    toks = {name: np.stack([np.stack([W.decode_tokens(w, name, b, h) for h in range(nh)], axis=1)
                            for b in batches]) for name, nh in (("q", w.n_q_heads), ("k", w.n_kv_heads),
                                                                ("v", w.n_kv_heads))}
    dq, dk, dv = (H.to_device(toks[x], w) for x in ("q", "k", "v"))        # [B, steps, H, d]
    outs, sels = [], []
    H.log(f"[{label}] GPU decode steps")
    for s in range(steps):
        o, sel = binding.decode_step(dq[:, s].contiguous(), dk[:, s].contiguous(), dv[:, s].contiguous(),
                                     kc, vc, pyr, n0 + s, K, out_dtype=torch.float32)
        outs.append(o.cpu().numpy())
        sels.append(sel.cpu().numpy())
    torch.cuda.synchronize()
    # incremental pyramid == rebuild, bit for bit (valid nodes of the final length)
    rebuilt = binding.build_pyramid(kc, n=cap, capacity=cap).cpu().numpy()
    got = pyr.cpu().numpy()
    for bi in range(B):
        for kvh in range(w.n_kv_heads):
            for a, r in zip(_pyramid_levels(got[bi, kvh], cap, cap), _pyramid_levels(rebuilt[bi, kvh], cap, cap)):
                np.testing.assert_array_equal(a, r)
    units = check_units if check_units is not None else [(bi, h) for bi in range(B) for h in range(w.n_kv_heads)]
    n_bad = n_total = 0
    worst = (0.0, 0.0)
    tol_abs, tol_rel = H.attn_tolerance(w)
    for bi, kvh in units:
        H.log(f"[{label}] oracle decode unit b={batches[bi]} kvh={kvh}")
        st = oracle.DecodeState(H.host_values(k0[bi, :, kvh]).astype(np.float64),
                                H.host_values(v0[bi, :, kvh]).astype(np.float64), capacity=cap)
        for s in range(steps):
            qh = toks["q"][bi, s, kvh * G:(kvh + 1) * G].astype(np.float64)
            osel, ogap, oo, _ = st.step(qh, toks["k"][bi, s, kvh], toks["v"][bi, s, kvh], K)
            gsel = sels[s][bi, kvh]
            n_total += 1
            if not np.array_equal(gsel, osel):
                assert ogap < H.GAP_LIMIT, (label, bi, kvh, s, gsel.tolist(), osel.tolist(), ogap)
                n_bad += 1
                continue
            ma, rl = H.attn_errors(outs[s][bi, kvh * G:(kvh + 1) * G], oo)
            worst = (max(worst[0], ma), max(worst[1], rl))
            assert ma <= tol_abs and rl <= tol_rel, (label, bi, kvh, s, ma, rl)
    if counts is None:
        H.assert_mismatch_budget(n_bad, n_total, label)
    else:
        counts.append((n_bad, n_total))
    H.log(f"[{label}] decode attention max-abs {worst[0]:.3g} rel-L2 {worst[1]:.3g}")


def test_decode_crosses_leaf_and_level_boundaries():
    # 1000 keys = 16 leaves (a power of two): the first step adds leaf 16 and a new root level
    w = W.WORKLOADS["decode_b64_ctx131072"].with_(name="dec_small", n_q_heads=8, n_kv_heads=2, top_k=4,
                                                  decode_steps=130, seed=50)
    run_decode(w, [0, 1], 1024 - 24, 130, "decode_small")


def test_decode_fp32_and_wide_group():
    w = W.WORKLOADS["tiny_f32_n1024"].with_(name="dec_f32", decode_steps=70, seed=51)
    run_decode(w, [0], 200, 70, "decode_f32_g4")
    w16 = W.WORKLOADS["decode_b64_ctx131072"].with_(name="dec_g16", n_q_heads=16, n_kv_heads=1, top_k=8,
                                                    decode_steps=40, seed=52)
    run_decode(w16, [0], 3000, 40, "decode_bf16_g16_k8")


def test_decode_from_a_single_key():
    w = W.WORKLOADS["decode_b64_ctx131072"].with_(name="dec_one", n_q_heads=4, n_kv_heads=1, top_k=2,
                                                  decode_steps=140, seed=53)
    run_decode(w, [0], 1, 140, "decode_from_one_key")


@pytest.mark.timeout(1200)
def test_decode_full_launch_b64(oracle_workers):
    """The 131072-token decode workload as the bench launches it: 64 sequences x 8 KV heads in every
    step, all 256 steps, head-major caches.  Sequences 0, 31 and 63 hold the seeded contexts and tokens and are checked
    on every KV head and step against the oracle (run in the forked pool); the other sequences are
    filled on the device.  The incremental pyramid equals a rebuild bit for bit for all 64."""
    import oracle_pool

    w = W.WORKLOADS["decode_b64_ctx131072"]
    B, n0, S, Hq, Hkv, d, G, K = (w.batch, w.seq_len, w.decode_steps, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                  w.group, w.top_k)
    checked = [0, 31, 63]
    cap = n0 + S
    pending = oracle_workers.map_async(oracle_pool.decode_unit, [(w, b, h, n0, S) for b in checked
                                                                  for h in range(Hkv)])
    H.log(f"[decode_b64] caches B={B} cap={cap} Hkv={Hkv} d={d}; checked sequences {checked}")
    gen = torch.Generator(device=H.DEV)
    gen.manual_seed(4)
    # head-major caches viewed as [B, cap, Hkv, d], the layout the bench times
    kc = torch.randn((B, Hkv, cap, d), generator=gen, device=H.DEV, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    vc = torch.randn((B, Hkv, cap, d), generator=gen, device=H.DEV, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    qs = torch.randn((S, B, Hq, d), generator=gen, device=H.DEV, dtype=torch.bfloat16)
    ks = torch.randn((S, B, Hkv, d), generator=gen, device=H.DEV, dtype=torch.bfloat16)
    vs = torch.randn((S, B, Hkv, d), generator=gen, device=H.DEV, dtype=torch.bfloat16)
    _, k0, v0 = W.prefill_inputs(w.with_(seq_len=n0), batches=checked, bits=True, with_q=False)
    for i, b in enumerate(checked):
        kc[b, :n0] = H.to_device(k0[i], w)
        vc[b, :n0] = H.to_device(v0[i], w)
        for name, dst, nh in (("q", qs, Hq), ("k", ks, Hkv), ("v", vs, Hkv)):
            host = np.stack([W.decode_tokens(w, name, b, h) for h in range(nh)], axis=1)   # [S, nh, d]
            dst[:, b] = H.to_device(host, w)
    del k0, v0
    pyr = binding.build_pyramid(kc, n=n0, capacity=cap)
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=H.DEV)
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device=H.DEV)
    idx = torch.tensor(checked, device=H.DEV)
    outs, sels = [], []
    H.log(f"[decode_b64] GPU decode steps")
    for s in range(S):
        binding.decode_step(qs[s], ks[s], vs[s], kc, vc, pyr, n0 + s, K, out=o, sel_out=sel)
        outs.append(o.index_select(0, idx).cpu().numpy())
        sels.append(sel.index_select(0, idx).cpu().numpy())
    rebuilt = binding.build_pyramid(kc, n=cap, capacity=cap)
    torch.cuda.synchronize()
    assert torch.equal(pyr, rebuilt), "incremental pyramid differs from a rebuild"
    del kc, vc, rebuilt, pyr
    torch.cuda.empty_cache()
    H.log(f"[decode_b64] waiting for the oracle")
    n_bad = n_total = 0
    worst = (0.0, 0.0)
    tol_abs, tol_rel = H.attn_tolerance(w)
    for b, kvh, osel, ogap, oo in pending.get():
        i = checked.index(b)
        for s in range(S):
            n_total += 1
            if not np.array_equal(sels[s][i, kvh], osel[s]):
                assert ogap[s] < H.GAP_LIMIT, (b, kvh, s, sels[s][i, kvh].tolist(), osel[s].tolist(), ogap[s])
                n_bad += 1
                continue
            ma, rl = H.attn_errors(outs[s][i, kvh * G:(kvh + 1) * G], oo[s])
            worst = (max(worst[0], ma), max(worst[1], rl))
            assert ma <= tol_abs and rl <= tol_rel, (b, kvh, s, ma, rl)
    assert n_total == len(checked) * Hkv * S
    H.assert_mismatch_budget(n_bad, n_total, "decode_b64")
    H.log(f"[decode_b64] attention max-abs {worst[0]:.3g} rel-L2 {worst[1]:.3g} over {n_total} (unit, step)s")
