"""A pool of CPU processes that runs the fp64 oracle over every token of the full-size workloads.

Test infrastructure: the pool is forked by tests/conftest.py when the session starts, before
anything touches the GPU, and the parity tests hand it chunks of query tokens.  Each worker draws
its own inputs from the seeded workload recipe (the same bytes the GPU path receives) and keeps
the (b, kvh) unit it last drew; nothing computed on the GPU ever enters the oracle.
"""
from __future__ import annotations

import os

import numpy as np

_CACHE: dict = {}


def worker_count() -> int:
    """One worker per host core, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)


def make_pool():
    """Fork the pool (call only from a process that has not initialised the GPU)."""
    import multiprocessing as mp

    return mp.get_context("fork").Pool(worker_count(), initializer=_init)


def _unit(spec, b: int, kvh: int, with_q: bool = True):
    """Float64 K, V, pyramid and the group's float32 queries of one (b, kvh), drawn once per worker."""
    from hierarchical_top_selection_amd import workloads as W
    from oracle import pisa as oracle

    key = (spec, b, kvh, with_q)
    if _CACHE.get("key") != key:
        _CACHE.clear()
        w = spec
        G = w.group
        k = W.draw(w, "k", b, kvh).astype(np.float64)
        v = W.draw(w, "v", b, kvh).astype(np.float64)
        q = np.stack([W.draw(w, "q", b, kvh * G + c) for c in range(G)], axis=1) if with_q else None
        _CACHE.update(key=key, k=k, v=v, q=q, pyr=oracle.build_pyramid(k))
    return _CACHE


def prefill_chunk(task):
    """Oracle selection, boundary record, leaf scores of the selected leaves and attention output
    for the tokens ``ts`` of one (b, kvh) unit.

    ``task`` = (workload, b, kvh, token positions, K).  Returns (b, kvh, ts, sel [T, K] int32,
    gap [T], sel_u [T, K] float64 (-inf on padding), o [T, G, d] float32, row LSE [T, G]).
    """
    from oracle import pisa as oracle

    spec, b, kvh, ts, K = task
    u = _unit(spec, b, kvh)
    ts = np.asarray(ts, dtype=np.int64)
    parts = [_prefill_part(u, ts[i:i + 32], K) for i in range(0, len(ts), 32)]   # bounded gathers
    sel, gap, sel_u, o, lse = (np.concatenate([p[i] for p in parts]) for i in range(5))
    return b, kvh, ts, sel, gap, sel_u, o, lse


def _prefill_part(u, ts, K):
    from oracle import pisa as oracle

    q = u["q"][ts].astype(np.float64)
    sel, gap, rec = oracle.route(q, u["k"], u["pyr"], ts, K, record=True)
    o, lse, _ = oracle.attention(q, u["k"], u["v"], sel, ts)
    # scores of the selected leaves, in the ascending order of ``sel``
    cand, cu = rec["leaf_cand"], rec["leaf_u"]
    match = (sel[:, :, None] == cand[:, None, :]) & (sel[:, :, None] >= 0)        # [T, K, candidates]
    sel_u = np.take_along_axis(cu, np.argmax(match, axis=2), axis=1)
    sel_u = np.where(sel >= 0, sel_u, -np.inf)
    for r, slot in zip(*np.nonzero((sel >= 0) & ~np.isfinite(sel_u))):
        # a leaf level kept whole is not scored by the routing: its exact leaf LSE, summed over heads
        sel_u[r, slot] = float(np.sum(oracle.leaf_lse(q[r], u["k"], int(sel[r, slot]), int(ts[r]))))
    return sel.astype(np.int32), gap, sel_u, o.astype(np.float32), lse


def decode_unit(task):
    """All decode steps of one (b, kvh) unit on the oracle.  ``task`` = (workload, b, kvh, context
    length, steps); returns (b, kvh, sel [S, K] int32, gap [S], o [S, G, d] float32)."""
    from hierarchical_top_selection_amd import workloads as W
    from oracle import pisa as oracle

    w, b, kvh, n0, steps = task
    G, K = w.group, w.top_k
    ctx = w.with_(seq_len=n0)
    st = oracle.DecodeState(W.draw(ctx, "k", b, kvh).astype(np.float64),
                            W.draw(ctx, "v", b, kvh).astype(np.float64), capacity=n0 + steps)
    qs = np.stack([W.decode_tokens(w, "q", b, kvh * G + c) for c in range(G)], axis=1)      # [S, G, d]
    ks, vs = W.decode_tokens(w, "k", b, kvh), W.decode_tokens(w, "v", b, kvh)
    sels, gaps, outs = [], [], []
    for s in range(steps):
        sel, gap, o, _ = st.step(qs[s].astype(np.float64), ks[s], vs[s], K)
        sels.append(sel)
        gaps.append(gap)
        outs.append(o)
    return b, kvh, np.array(sels, dtype=np.int32), np.array(gaps), np.array(outs, dtype=np.float32)
