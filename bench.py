#!/usr/bin/env python3
"""Prefill throughput of the PISA hot path on one MI355X.

One step = build the key pyramid, select the top-K leaf blocks of every query
token (routing, clustering, exact leaf LSE, top-K) and run block-sparse
attention over them, for the whole batch of one workload, with inputs already
resident in HBM.  Prints ONE JSON line (see the design notes for the fields).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload prefill_n262144]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from hierarchical_top_selection_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


# ----------------------------------------------------------------------------- CPU baseline (oracle)
_CPU = {}


def _cpu_init(q, k, v, pyr, K):
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)
    _CPU.update(q=q, k=k, v=v, pyr=pyr, K=K)


def _cpu_chunk(ts):
    from oracle import pisa as oracle

    ts = np.asarray(ts)
    sel, _ = oracle.route(_CPU["q"][ts], _CPU["k"], _CPU["pyr"], ts, _CPU["K"])
    oracle.attention(_CPU["q"][ts], _CPU["k"], _CPU["v"], sel, ts)
    return len(ts)


def cpu_baseline(w: W.Workload, seconds: float) -> dict:
    """The fp64 oracle on a time-bounded sample of (b=0, kvh=0) tokens, extrapolated to the workload."""
    import multiprocessing as mp

    from oracle import pisa as oracle

    G = w.group
    q = np.stack([W.draw(w, "q", 0, h) for h in range(G)], axis=1).astype(np.float64)
    k = W.draw(w, "k", 0, 0).astype(np.float64)
    v = W.draw(w, "v", 0, 0).astype(np.float64)
    t0 = time.perf_counter()
    pyr = oracle.build_pyramid(k)
    t_pyr = time.perf_counter() - t0
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    order = np.random.default_rng(12345).permutation(w.seq_len)
    chunks = [np.sort(order[i:i + 16]) for i in range(0, w.seq_len, 16)]
    done = 0
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_cpu_init, initargs=(q, k, v, pyr, w.top_k)) as pool:
        t0 = time.perf_counter()
        for n in pool.imap_unordered(_cpu_chunk, chunks):
            done += n
            if time.perf_counter() - t0 > seconds:
                break
        elapsed = time.perf_counter() - t0
        pool.terminate()
    units = w.batch * w.n_kv_heads
    full_s = units * t_pyr + units * w.seq_len * elapsed / done
    return {"value": w.batch * w.seq_len / full_s, "unit": "tokens/s", "cores": workers,
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done} query tokens of (b=0, kvh=0) drawn uniformly from the {w.seq_len}-token sequence "
                      f"(fp64 NumPy routing, leaf LSE, top-K and attention) in {elapsed:.1f} s on {workers} "
                      f"processes, plus one pyramid build ({t_pyr:.2f} s); extrapolated to "
                      f"{units} x {w.seq_len} tokens"}


# ----------------------------------------------------------------------------- GPU
def _device_inputs(w: W.Workload):
    import torch

    q, k, v = W.prefill_inputs(w, bits=True)

    def dev(x):
        if w.dtype == "f32":
            return torch.from_numpy(x).to("cuda:0")
        return torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)

    return dev(q), dev(k), dev(v)


_INPUTS = {}   # device Q and K of each workload run, reused by the selection sweep


def attention_flops(sel, n: int, group: int, d: int) -> float:
    """4 d flops per (query head, valid key): keys of the selected blocks at positions <= t."""
    import torch

    t = torch.arange(n, device=sel.device, dtype=torch.int64).view(1, 1, n, 1)
    j = sel.to(torch.int64)
    valid = torch.clamp(torch.minimum(t - 64 * j + 1, torch.full_like(j, 64)), min=0)
    valid = torch.minimum(valid, torch.clamp(n - 64 * j, min=0))
    valid = torch.where(j >= 0, valid, torch.zeros_like(valid))
    return float(valid.sum().item()) * group * 4.0 * d


def level_sizes(n: int) -> list[int]:
    """Nodes per pyramid level for n keys, leaves first: ceil(n / 64), then ceil(/2) down to 1."""
    sizes = [-(-n // 64)]
    while sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // 2))
    return sizes


def compulsory_bytes(w: W.Workload) -> dict:
    """HBM bytes each prefill kernel must move at the least: every input it reads once, every
    output it writes once (per launch; the attention kernel's per call)."""
    B, N, G, d, K = w.batch, w.seq_len, w.group, w.head_dim, w.top_k
    bh, s, width = w.batch * w.n_kv_heads, (2 if w.dtype == "bf16" else 4), 2 * K
    sizes = level_sizes(N)
    m1, nodes = sizes[0], sum(sizes)
    windows = -(-N // (512 if N <= 65536 else 1024))
    slots = bh * N * width * 4
    q_bytes = bh * N * G * d * s
    packed = bh * m1 * 64 * d * 2
    return {
        "pyramid_leaves_kernel": bh * N * d * s + bh * sum(sizes[:4]) * d * 4,
        "pyramid_top_kernel": bh * (sizes[3] if len(sizes) > 3 else 0) * d * 4 + bh * sum(sizes[4:]) * d * 4,
        "split_summaries_kernel": bh * nodes * d * 4 + bh * sum(-(-m // 2) for m in sizes) * 8 * d,
        "route_kernel": q_bytes + (bh * N * G * d * 2 if w.dtype == "bf16" else 0) + slots,
        "route_prefilter_kernel": q_bytes + bh * N * G * d * 2 + slots,
        "cluster_kernel": 2 * slots + bh * windows * (m1 + 1) * 4,
        "pack_blocks_kernel": bh * N * d * 2 + packed,
        "leaf_lse_kernel": bh * N * G * d * 2 + packed + 2 * slots,
        "topk_kernel": 2 * slots + bh * N * K * 4,
        "attention_pack": 2 * (bh * N * d * 2 + packed),
    }


def decode_step_bytes(w: W.Workload, n_ctx: int) -> int:
    """HBM bytes one decode step must move at the least, for every (b, kvh) unit, with the new token
    at position n_ctx (all nodes valid): the children summaries of every scored level, the raw keys of
    the candidate leaves, the values of the K selected blocks, the queries and outputs, the appended
    key and value, and the refreshed leaf with its ancestor path.  Candidate counts take the upper
    bound min(2 * kept, level size) at every level."""
    d, G, K, s = w.head_dim, w.group, w.top_k, (2 if w.dtype == "bf16" else 4)
    sizes = level_sizes(n_ctx + 1)
    per = 0
    cand = 1                                            # the root
    for lvl in range(len(sizes), 1, -1):                # children live at level lvl - 1
        kids = min(2 * min(cand, K), sizes[lvl - 2])
        if cand > K:
            per += min(2 * cand, sizes[lvl - 2]) * d * 4  # children summaries of every candidate
        cand = kids
    per += cand * 64 * d * s                            # raw keys of the candidate leaves
    per += min(K, sizes[0]) * 64 * d * s                # values of the selected blocks
    per += G * d * s + G * d * s                        # query rows in, output rows out
    per += 2 * d * s * 2                                # new key and value, read and written
    per += 64 * d * s + 2 * len(sizes) * d * 4          # the leaf's keys, ancestor path read and written
    return per * w.batch * w.n_kv_heads


# kernels that choose and build the attention passes' token order (up to 16384 leaf blocks)
ORDER_KERNELS = ["order_clear_kernel", "order_share_kernel", "order_hist_kernel", "order_keys_kernel",
                 "order_prefix_kernel", "order_keyscan_kernel", "order_scatter_kernel"]


def stage_kernels(w: W.Workload) -> dict:
    """Kernels each entry point launches, in launch order, for a prefill workload (their names)."""
    bf16 = w.dtype == "bf16"
    levels = len(level_sizes(w.seq_len))
    return {
        "pyramid": ["pyramid_leaves_kernel"] + (["pyramid_top_kernel"] if levels > 4 else []),
        "select": (["split_summaries_kernel", "route_prefilter_kernel"] if bf16 else ["route_kernel"]) + ["cluster_kernel"]
                  + (["pack_blocks_kernel"] if bf16 else []) + ["leaf_lse_kernel", "topk_kernel"],
        "attention": (["pack_blocks_kernel"] + (ORDER_KERNELS if level_sizes(w.seq_len)[0] <= 16384 else [])
                      + ["attention_bf16_kernel", "attention_bf16_kernel"] if bf16 else ["attention_f32_kernel"]),
    }


def run_workload(w: W.Workload, steps: int, warmup: int) -> dict:
    """Timed prefill steps.  Besides the host wall clock and the events around each entry point,
    the library records one event after every kernel it enqueues (pisa_stage_events), so every
    kernel's duration is measured on the stream it runs on."""
    import torch

    from hierarchical_top_selection_amd import binding

    q, k, v = _device_inputs(w)
    _INPUTS[w.name] = (q, k, v)
    B, N, Hq, d = q.shape
    K = w.top_k
    pyr = torch.empty((B, w.n_kv_heads, binding.pyramid_nodes(N), d), dtype=torch.float32, device=q.device)
    cfg = binding.make_cfg(B, N, Hq, w.n_kv_heads, d, K, q.dtype)
    ws = torch.empty(binding.select_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
    ws_attn = torch.empty(max(1, binding.attn_workspace_bytes(cfg)), dtype=torch.uint8, device=q.device)
    sel = torch.empty((B, w.n_kv_heads, N, K), dtype=torch.int32, device=q.device)
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)   # fp32 attention output
    names = stage_kernels(w)
    calls = ("pyramid", "select", "attention")

    def step(ev=None):
        # ev: per call, [start, one event per kernel]
        if ev is not None:
            ev["pyramid"][0].record()
            binding.stage_events(ev["pyramid"][1:])
        binding.build_pyramid(k, out=pyr)
        if ev is not None:
            ev["select"][0].record()
            binding.stage_events(ev["select"][1:])
        binding.select_blocks(q, k, pyr, K, workspace=ws, out=sel)
        if ev is not None:
            ev["attention"][0].record()
            binding.stage_events(ev["attention"][1:])
        binding.sparse_attn_fwd(q, k, v, sel, out=o, workspace=ws_attn)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [{c: [torch.cuda.Event(enable_timing=True) for _ in range(1 + len(names[c]))] for c in calls}
              for _ in range(steps)]
    for ev in events:                      # create the events before the timed region
        for lst in ev.values():
            for e in lst:
                e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    call_ms = {c: sum(ev[c][0].elapsed_time(ev[c][-1]) for ev in events) / steps for c in calls}
    kernel_ms = {c: [sum(ev[c][i].elapsed_time(ev[c][i + 1]) for ev in events) / steps
                     for i in range(len(names[c]))] for c in calls}
    flops = attention_flops(sel, N, w.group, d)
    cand = ws[:B * w.n_kv_heads * N * 2 * K * 4].view(torch.int32).view(B, w.n_kv_heads, N, 2 * K)
    leaf_flops = attention_flops(cand, N, w.group, d) / 2.0          # Q K^T only: 2 d per (head, key)
    return {"workload": w, "ms_per_step": wall_ms, "pyramid_ms": call_ms["pyramid"], "select_ms": call_ms["select"],
            "attn_ms": call_ms["attention"], "tokens_per_s": B * N / (wall_ms / 1e3), "attn_flops": flops,
            "leaf_flops": leaf_flops, "kernel_names": names, "kernel_ms": kernel_ms}


def selection_sweep(q, k, n_kv_heads: int, K: int = 8, reps: int = 5, w: W.Workload | None = None,
                    longer=(524288, 1000000)) -> dict:
    """Selection latency, hierarchical vs single-level, on prefixes N = 4K .. full of one input,
    then at the `longer` lengths on device-drawn inputs of the same recipe (`W.device_prefill_inputs`).

    Both sides build the key pyramid (the flat scan reads its leaf means) and then
    select K leaves per token: `select_blocks` (routing + exact leaf LSE + top-K)
    against `select_flat` (every valid leaf scored by its mean key).  Median of `reps`
    timed runs after one warm-up, HIP events on the current stream.
    """
    import torch

    from hierarchical_top_selection_amd import binding

    B, N, Hq, d = q.shape
    ns = [n for n in (4096, 8192, 16384, 32768, 65536, 131072, 262144) if n <= N]
    longer = [n for n in longer if n > N] if w is not None else []
    out = {"K": K, "n": ns + longer, "device_drawn_from": longer[0] if longer else None,
           "pisa_select_ms": [], "flat_select_ms": [], "flat_over_pisa": []}
    for n in ns + longer:
        if n in longer:
            qn, kn = W.device_prefill_inputs(w, n)
        else:
            qn, kn = q[:, :n], k[:, :n]
        cfg = binding.make_cfg(B, n, Hq, n_kv_heads, d, K, q.dtype)
        ws_h = torch.empty(binding.select_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
        ws_f = torch.empty(binding.flat_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
        pyr = torch.empty((B, n_kv_heads, binding.pyramid_nodes(n), d), dtype=torch.float32, device=q.device)
        sel = torch.empty((B, n_kv_heads, n, K), dtype=torch.int32, device=q.device)
        runs = {
            "pisa_select_ms": lambda: (binding.build_pyramid(kn, out=pyr),
                                       binding.select_blocks(qn, kn, pyr, K, workspace=ws_h, out=sel)),
            "flat_select_ms": lambda: (binding.build_pyramid(kn, out=pyr),
                                       binding.select_flat(qn, pyr, n_kv_heads, K, workspace=ws_f, out=sel)),
        }
        for key, fn in runs.items():
            fn()
            times = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            out[key].append(sorted(times)[len(times) // 2])
        out["flat_over_pisa"].append(out["flat_select_ms"][-1] / out["pisa_select_ms"][-1])
        del ws_h, ws_f, pyr, sel, qn, kn
        torch.cuda.empty_cache()
    r = out["flat_over_pisa"]
    cross = next((i for i in range(1, len(r)) if r[i - 1] < 1.0 <= r[i]), None)
    out["crossover_between"] = None if cross is None else [out["n"][cross - 1], out["n"][cross]]
    return out


def variant_selection(q, k, n_kv_heads: int, K: int, reps: int = 5) -> dict:
    """Selection latency (pyramid + select_blocks) of each candidate score on one input, median of reps."""
    import torch

    from hierarchical_top_selection_amd import binding

    B, N, Hq, d = q.shape
    cfg = binding.make_cfg(B, N, Hq, n_kv_heads, d, K, q.dtype)
    ws = torch.empty(binding.select_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
    pyr = torch.empty((B, n_kv_heads, binding.pyramid_nodes(N), d), dtype=torch.float32, device=q.device)
    sel = torch.empty((B, n_kv_heads, N, K), dtype=torch.int32, device=q.device)
    out = {"K": K}
    for score in ("lse", "mean", "mean_var"):
        def fn():
            binding.build_pyramid(k, out=pyr)
            binding.select_blocks(q, k, pyr, K, workspace=ws, out=sel, score=score)
        fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[f"{score}_select_ms"] = sorted(times)[len(times) // 2]
    return out


def run_backward(q, k, v, n_kv_heads: int, K: int, reps: int = 5) -> dict:
    """Attention gradients of one prefill: selection and forward once (untimed), then the median
    of `reps` timed calls of sparse_attn_bwd (HIP events on the current stream).

    dO is drawn on the device (seeded torch generator, N(0,1), float32); the forward output is
    float32.  Work counts valid (head, key) pairs like the forward: the dq pass does 3 products
    and the dk/dv pass 4, 14 d flops per pair in all.
    """
    import torch

    from hierarchical_top_selection_amd import binding

    B, N, Hq, d = q.shape
    G = Hq // n_kv_heads
    pyr = binding.build_pyramid(k)
    sel = binding.select_blocks(q, k, pyr, K)
    o, lse = binding.sparse_attn_fwd(q, k, v, sel, return_lse=True, out_dtype=torch.float32)
    gen = torch.Generator(device=q.device)
    gen.manual_seed(7)
    dout = torch.randn(o.shape, generator=gen, device=q.device, dtype=torch.float32)
    cfg = binding.make_cfg(B, N, Hq, n_kv_heads, d, K, q.dtype)
    ws = torch.empty(binding.attn_bwd_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)

    def fn():
        binding.sparse_attn_bwd(q, k, v, sel, o, lse, dout, workspace=ws, dq=dq, dk=dk, dv=dv)

    fn()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    flops = attention_flops(sel, N, G, d) * 14.0 / 4.0
    out = {"K": K, "bwd_ms": ms, "tokens_per_s": B * N / (ms / 1e3), "tflops": flops / (ms * 1e-3) / 1e12,
           "workspace_gb": ws.numel() / 1e9, "data": "dO: device-drawn N(0,1), seeded torch generator"}
    del ws, dq, dk, dv, dout, o, lse, sel, pyr
    return out


def _mean_present(xs):
    xs = [x for x in xs if x is not None]
    return sum(xs) / len(xs) if xs else None


def selection_quality(q, k, n_kv_heads: int, K: int, tokens: int = 256, seed: int = 5) -> dict:
    """Recall@K against the exact flat top-K and retained attention mass of each selector.

    The hierarchical selection with each candidate score and the flat mean-key scan select
    on the full input; `quality.selection_quality` then scores `tokens` sampled positions
    t >= 2 K C (where a choice exists) against the exact per-leaf LSE, spread over the
    KV heads.  Not timed: a measurement of what is selected, reported beside the speed.
    """
    import numpy as np
    import torch

    from hierarchical_top_selection_amd import binding, quality

    B, N, Hq, d = q.shape
    pyr = binding.build_pyramid(k)
    sels = {f"pisa_{score}": binding.select_blocks(q, k, pyr, K, score=score) for score in ("lse", "mean", "mean_var")}
    sels["flat_mean"] = binding.select_flat(q, pyr, n_kv_heads, K)
    torch.cuda.synchronize()
    heads = min(n_kv_heads, 4)
    rng = np.random.default_rng(seed)
    acc = {}
    for kvh in range(heads):
        ts = np.sort(rng.choice(np.arange(2 * K * 64, N), tokens // heads, replace=False))
        r = quality.selection_quality(q, k, sels, ts, K, kvh=kvh)
        for name, m in r.items():
            a = acc.setdefault(name, {key: [] for key in m})
            for key, val in m.items():
                a[key].append(val)
    out = {"K": K, "tokens": (tokens // heads) * heads, "kv_heads": heads, "position_bins": 4}
    for name, a in acc.items():
        out[name] = {"recall": float(np.mean(a["recall"])), "mass": float(np.mean(a["mass"])),
                     **{key: [_mean_present([x[i] for x in a[key]]) for i in range(4)]
                        for key in ("recall_by_position", "mass_by_position")}}
    del sels, pyr
    return out


def run_decode(w: W.Workload, warmup_passes: int = 1) -> dict:
    """Decode throughput: `decode_steps` steps of every sequence after a prebuilt context.

    The 2 x 17 GB bf16 caches are drawn on the device with a seeded torch generator
    (N(0, 1), like the workload's recipe; drawing them on the host would take minutes) and laid
    out head-major.
    One untimed pass of all steps runs first; the pyramid is then rebuilt for the
    context length, so the timed pass starts from the same state.
    """
    import torch

    from hierarchical_top_selection_amd import binding

    B, n0, Hq, Hkv, d, K, S = w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.top_k, w.decode_steps
    cap = n0 + S
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(w.seed)
    # head-major caches ([B, Hkv, cap, d] in memory, viewed as [B, cap, Hkv, d]): each (sequence,
    # KV head) keeps its keys and values contiguous, so a leaf block is one 16 KB run
    kc = torch.randn((B, Hkv, cap, d), generator=gen, device="cuda:0", dtype=torch.bfloat16).permute(0, 2, 1, 3)
    vc = torch.randn((B, Hkv, cap, d), generator=gen, device="cuda:0", dtype=torch.bfloat16).permute(0, 2, 1, 3)
    qs = torch.randn((S, B, Hq, d), generator=gen, device="cuda:0", dtype=torch.bfloat16)
    ks = kc[:, n0:].permute(1, 0, 2, 3).contiguous()          # the appended tokens, [S, B, Hkv, d]
    vs = vc[:, n0:].permute(1, 0, 2, 3).contiguous()
    pyr = torch.empty((B, Hkv, binding.pyramid_nodes(cap), d), dtype=torch.float32, device="cuda:0")
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda:0")
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda:0")

    def one_pass(ev=None):
        binding.build_pyramid(kc, n=n0, capacity=cap, out=pyr)
        if ev is not None:
            ev[0].record()
        for s in range(S):
            binding.decode_step(qs[s], ks[s], vs[s], kc, vc, pyr, n0 + s, K, out=o, sel_out=sel)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup_passes):
        one_pass()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    one_pass(ev)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    del kc, vc
    torch.cuda.empty_cache()
    ms = total_ms / S
    step_bytes = sum(decode_step_bytes(w, n0 + i) for i in range(S)) / S
    return {"tokens_per_s": B * S / (total_ms * 1e-3), "ms_per_step": ms, "steps": S, "batch": B,
            "context": n0, "data": "synthetic: device-drawn N(0,1), seeded torch generator",
            "roofline": {"bound": "hbm", "bytes_per_step": step_bytes, "achieved": step_bytes / (ms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


# HBM-side traffic per launch of each kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes scaled by
# a plain device copy (committed under profiles/).  A kernel's figure is reported only while its
# sources are the ones the counters were taken on; otherwise it is null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_n262144_traffic.md")
_COMMON = ("kernels.h", "pisa_device.h")
KERNEL_SOURCES = {
    "pyramid_leaves_kernel": ("pyramid.hip", "pyramid_dev.h") + _COMMON,
    "pyramid_top_kernel": ("pyramid.hip", "pyramid_dev.h") + _COMMON,
    "split_summaries_kernel": ("route.hip",) + _COMMON,
    "route_kernel": ("route.hip",) + _COMMON,
    "route_prefilter_kernel": ("route.hip",) + _COMMON,
    "cluster_kernel": ("cluster.hip",) + _COMMON,
    "pack_blocks_kernel": ("pack.hip",) + _COMMON,
    "leaf_lse_kernel": ("leaf_lse.hip",) + _COMMON,
    "topk_kernel": ("topk.hip",) + _COMMON,
    "attention_bf16_kernel": ("attention.hip",) + _COMMON,
}


def source_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "hierarchical_top_selection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_traffic(workload: str) -> dict:
    """{kernel: HBM-side bytes per launch} for the kernels whose committed counters match the current
    sources (record lines `traffic: <kernel> fetch=<bytes> write=<bytes> sha256=<hex>`)."""
    if workload != "prefill_n262144" or not os.path.exists(TRAFFIC_FILE):
        return {}
    out = {}
    for name, fetch, write, sha in re.findall(r"^traffic: (\w+) fetch=(\d+) write=(\d+) sha256=([0-9a-f]+)\s*$",
                                              open(TRAFFIC_FILE).read(), re.M):
        if name in KERNEL_SOURCES and sha == source_sha256(name):
            out[name] = int(fetch) + int(write)
    return out


def kernel_table(run: dict) -> list:
    """Per-kernel duration (HIP events on the launch stream), compulsory HBM bytes and their rate
    against the 8 TB/s peak, counter traffic where current, and the MFMA rate of the leaf scores."""
    w = run["workload"]
    need = compulsory_bytes(w)
    traffic = kernel_traffic(w.name)
    rows = []
    for call in ("pyramid", "select"):
        for name, ms in zip(run["kernel_names"][call], run["kernel_ms"][call]):
            row = {"kernel": name, "call": call, "ms": ms, "bytes": need[name],
                   "achieved_gbs": need[name] / (ms * 1e-3) / 1e9}
            row["frac"] = row["achieved_gbs"] / HBM_PEAK_GBS
            tr = traffic.get(name)
            row["traffic"] = tr
            row["traffic_frac"] = None if tr is None else tr / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
            if name == "leaf_lse_kernel":
                peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
                row["flops"] = run["leaf_flops"]
                row["mfma_frac"] = run["leaf_flops"] / (ms * 1e-3) / 1e12 / peak
            rows.append(row)
    return rows


def attention_roofline(run: dict) -> dict:
    """The attention kernel against the bf16 MFMA peak: valid-key flops of one call over the summed
    durations of its launches (one per pass), each timed with HIP events on the launch stream."""
    w = run["workload"]
    names, ms = run["kernel_names"]["attention"], run["kernel_ms"]["attention"]
    kernel = names[-1]
    launch_ms = [m for n, m in zip(names, ms) if n == kernel]
    tflops = run["attn_flops"] / (sum(launch_ms) * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    traffic = kernel_traffic(w.name).get(kernel)
    return {"kernel": kernel, "launches": len(launch_ms), "launch_ms": launch_ms, "bound": "mfma",
            "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak,
            "traffic": None if traffic is None else traffic * len(launch_ms)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_n262144")
    ap.add_argument("--also", default="prefill_n32768", help="comma-separated extra workloads to report")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode timing record")
    ap.add_argument("--no-quality", action="store_true", help="skip the selection-quality record")
    ap.add_argument("--no-backward", action="store_true", help="skip the attention-gradient record")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the hierarchical vs single-level selection sweep (K = 8, N = 4K .. the workload's N)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the decode record (for profiling it alone) and print it as one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times), for scaling HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; runs on more than one GPU are not supported "
              "(the design notes describe how it would shard)", file=sys.stderr)
        return 2
    if args.copy_calibration:
        import torch

        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "reads": src.numel() * 4, "writes": src.numel() * 4}))
        return 0
    if args.decode_only:
        print(json.dumps({"decode_b64_ctx131072": run_decode(W.WORKLOADS["decode_b64_ctx131072"])}))
        return 0
    w = W.WORKLOADS[args.workload]
    also = [x for x in args.also.split(",") if x and x != args.workload]
    # the oracle baselines run before any GPU use (their pools fork)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    cpu_extra = {} if args.no_cpu_baseline else {name: cpu_baseline(W.WORKLOADS[name], args.cpu_seconds)
                                                 for name in also}

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    main_run = run_workload(w, args.steps, args.warmup)
    extra = {}
    for name in also:
        r = run_workload(W.WORKLOADS[name], args.steps, args.warmup)
        extra[name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                       "pyramid_ms": r["pyramid_ms"], "select_ms": r["select_ms"], "attn_ms": r["attn_ms"],
                       "roofline": attention_roofline(r), "selection_roofline": kernel_table(r),
                       "cpu_baseline": cpu_extra.get(name)}
    if not args.no_sweep:
        q_main, k_main, _ = _INPUTS[w.name]
        extra["selection_sweep_k8"] = selection_sweep(q_main, k_main, w.n_kv_heads, K=8, w=w)
        extra["score_variants"] = variant_selection(q_main, k_main, w.n_kv_heads, w.top_k)
    if not args.no_backward:
        q_main, k_main, v_main = _INPUTS[w.name]
        extra["backward_" + w.name] = run_backward(q_main, k_main, v_main, w.n_kv_heads, w.top_k)
    if not args.no_quality:
        q_main, k_main, _ = _INPUTS[w.name]
        extra["selection_quality_k8"] = selection_quality(q_main, k_main, w.n_kv_heads, 8)
        for name in ("quality_diffuse_n65536", "quality_needles_n65536", "quality_runs_n65536"):
            rw = W.WORKLOADS[name]
            rq, rk, _ = _device_inputs(rw)
            extra[name] = selection_quality(rq, rk, rw.n_kv_heads, rw.top_k)
            del rq, rk
    _INPUTS.clear()
    if not args.no_decode:
        extra["decode_b64_ctx131072"] = run_decode(W.WORKLOADS["decode_b64_ctx131072"])
    line = {
        "metric": "prefill tokens/s (select+sparse attn)",
        "value": main_run["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block": w.block, "fanout": w.fanout,
                   "top_k": w.top_k, "parallelism": "single_gpu"},
        "pyramid_ms": main_run["pyramid_ms"],
        "select_ms": main_run["select_ms"],
        "attn_ms": main_run["attn_ms"],
        # the dominant kernel: attention_bf16_kernel, launched once per pass (even, then odd block
        # ids, for a float32 output); achieved and traffic are per call (both launches), flops count
        # valid keys only
        "roofline": attention_roofline(main_run),
        # every pyramid and selection kernel: duration, compulsory HBM bytes and their fraction of
        # 8 TB/s, counter traffic where current; the leaf scores also against the bf16 MFMA peak
        "selection_roofline": kernel_table(main_run),
        "cpu_baseline": cpu,
        "also": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
