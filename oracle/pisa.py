"""Float64 oracle for PISA: key pyramid, LSE routing, leaf top-K, sparse attention, decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
the smoke check and the benchmark's CPU baseline, never by the library.

Citations name sections of the paper-summary page "Block Sparse Attention
with Log-Linear Complexity" (Tang, Qin, Pan, Li, Liu):
  [Prereq/BSA]   Prerequisites, block sparse attention paragraph
  [Prereq/LSE]   Prerequisites, LogSumExp paragraph
  [Prereq/GQA]   Prerequisites, grouped-query attention paragraph
  [Core]         Core method (pyramid, routing, eq. 10-15, 16-20, 21)
  [Steps]        Method steps (pyramid mean, Stage 1 head sum eq. 22,
                 Stage 2 leaf LSE, decode update, attention on selected leaves)

Notation (the page's): level 0 = raw keys; level 1 = leaf blocks of C keys
(M_1 = ceil(n / C)); level l+1 pools g adjacent level-l nodes; the root is
the single node of level L.  Arrays here index levels from 1: ``pyr[0]`` is
level 1 (leaves), ``pyr[-1]`` the root level.

Readings where the pages are silent (each listed in the design notes):
  R1  Pyramid nodes are the unweighted mean of their (up to g) children, as
      printed; grouping is aligned at index 0; summaries are built once over
      all n keys and do not depend on the query.
  R2  Causal validity: node (l, i) is a candidate for query t only if its
      first token i * C * g**(l-1) <= t; scores use valid children only; the
      leaf LSE and attention use raw keys at positions <= t.  No forced blocks.
  R3  SelectK keeps min(K, |A|) candidates ordered by (score desc, index asc);
      levels with at most K candidates are kept whole and not scored.
  R4  The selected set is reported ascending, padded with -1 to K entries.
  R5  Attention is a softmax over the union of the selected blocks' keys at
      positions <= t, with the same 1/sqrt(d) scale as the scores.
  R6  Decode appends the new key/value at position n, updates the leaf of n
      and its ancestor path, then routes the new query with every key valid.
  R8  Score variants [Core: Taylor expansion of the LSE score into a mean and a
      variance correction; the PISA-1 / PISA-2 ablations]: "mean" (PISA-1)
      scores a candidate by the mean of its valid children's logits and
      "mean_var" (PISA-2) by that mean plus half their population variance;
      neither carries the log m term.  Both apply at every scored level,
      the leaf level included (raw keys <= t), with the same head sum.
  R7  The flat (single-level) baseline of the block-sparse framework scores
      every causally valid leaf j by its summary dot product q . k_bar_j *
      scale [Prereq/BSA, top-K block selection], with k_bar_j the leaf mean
      of the pyramid (built over the whole block, like every summary), sums
      the scores over the group's heads [Prereq/GQA] and keeps K by
      (score desc, index asc).
  R9  Gradients [Steps, attention on the selected leaves; the page calls the
      method trainable but gives no gradient treatment]: the gradient of the
      block-sparse attention output with the selected sets held fixed (the
      selection is piecewise constant in q and k, so no gradient flows
      through it).  Only the attention's dependence on q, k and v is
      differentiated; the routing scores carry none.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------- pyramid
def level_sizes(n: int, C: int = 64, g: int = 2) -> list[int]:
    """[M_1, M_2, ..., 1]: nodes per level for n keys [Core: pyramid of O(log N) levels]."""
    if n <= 0:
        return []
    sizes = [-(-n // C)]
    while sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // g))
    return sizes


def first_token(level: int, i, C: int = 64, g: int = 2):
    """Position of the first raw key covered by node i of ``level`` (level 1 = leaves) [R2]."""
    return i * C * g ** (level - 1)


def build_pyramid(k: np.ndarray, C: int = 64, g: int = 2) -> list[np.ndarray]:
    """Mean-pooled key pyramid [Steps: first step; Core: eq. 10-15].

    Level 1 node i is the mean of raw keys [iC, min((i+1)C, n)); a node of
    level l+1 is the mean of its children, k_bar^(l+1)_i = (1/|Ch_l(i)|) *
    sum_{r in Ch_l(i)} k_bar^(l)_r, with Ch_l(i) = {g*i, ..., g*i+g-1} cut to
    the level's size (R1).
    """
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    sizes = level_sizes(n, C, g)
    leaves = np.stack([k[i * C:min((i + 1) * C, n)].mean(axis=0) for i in range(sizes[0])])
    levels = [leaves]
    for m in sizes[1:]:
        prev = levels[-1]
        levels.append(np.stack([prev[g * i:min(g * i + g, prev.shape[0])].mean(axis=0)
                                for i in range(m)]))
    return levels


def update_pyramid(levels: list[np.ndarray], k: np.ndarray, n_new: int, C: int = 64,
                   g: int = 2) -> list[np.ndarray]:
    """Incremental pyramid update after key n_new-1 was appended [Steps: third step].

    Only the leaf holding the new key and that leaf's ancestor path are
    recomputed; a level that gains a node grows by one row, and a new root
    level appears when the old top level reaches two nodes.  Returns a new
    list (inputs are not modified).
    """
    k = np.asarray(k, dtype=np.float64)
    levels = [lv.copy() for lv in levels]
    pos = n_new - 1
    j = pos // C
    leaf = k[j * C:n_new].mean(axis=0)
    if not levels:
        levels = [leaf[None, :]]
    elif j == levels[0].shape[0]:
        levels[0] = np.vstack([levels[0], leaf[None, :]])
    else:
        levels[0][j] = leaf
    lvl, idx = 0, j
    while levels[lvl].shape[0] > 1:
        parent = idx // g
        kids = levels[lvl][g * parent:min(g * parent + g, levels[lvl].shape[0])]
        value = kids.mean(axis=0)
        if lvl + 1 == len(levels):
            levels.append(value[None, :])
        elif parent == levels[lvl + 1].shape[0]:
            levels[lvl + 1] = np.vstack([levels[lvl + 1], value[None, :]])
        else:
            levels[lvl + 1][parent] = value
        lvl, idx = lvl + 1, parent
    # a stale level above the new root cannot exist: levels only grow
    return levels


# ----------------------------------------------------------------------------- scores
def logsumexp(z: np.ndarray, axis: int = -1) -> np.ndarray:
    """log sum_j exp(z_j) along ``axis``, -inf where every entry is -inf [Prereq/LSE]."""
    m = np.max(z, axis=axis, keepdims=True)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = np.log(np.sum(np.exp(z - safe), axis=axis, keepdims=True)) + safe
    return np.squeeze(out, axis=axis)


SCORES = ("lse", "mean", "mean_var")


def child_score(z: np.ndarray, ok: np.ndarray, score: str = "lse") -> np.ndarray:
    """Score of a candidate from its children's logits ``z`` [..., c] (valid where ``ok``).

    "lse": log sum exp over the valid children [Core: eq. 21]; "mean" (PISA-1) and
    "mean_var" (PISA-2): mean, and mean plus half the population variance, of the
    valid children's logits [R8].  -inf when no child is valid.
    """
    if score == "lse":
        return logsumexp(np.where(ok, z, NEG_INF), axis=-1)
    m = ok.sum(axis=-1)
    zz = np.where(ok, z, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        mean = zz.sum(axis=-1) / m
        out = mean
        if score == "mean_var":
            dev = np.where(ok, z - mean[..., None], 0.0)
            out = mean + 0.5 * (dev * dev).sum(axis=-1) / m
        elif score != "mean":
            raise ValueError(f"unknown score {score!r}")
    return np.where(m > 0, out, NEG_INF)


def _select_k(u: np.ndarray, ids: np.ndarray, K: int):
    """Per row: order candidates by (u desc, id asc) [R3]; returns the order and the K-th gap.

    ``u`` is -inf and ``ids`` -1 on padding.  The gap is u_(K) - u_(K+1) of
    the sorted row (inf when the row has at most K valid entries).
    """
    key_ids = np.where(ids >= 0, ids, np.iinfo(np.int64).max)
    order = np.lexsort((key_ids, -u), axis=-1)
    su = np.take_along_axis(u, order, axis=-1)
    if u.shape[1] > K:
        with np.errstate(invalid="ignore"):           # -inf - -inf on rows with <= K valid entries
            gap = su[:, K - 1] - su[:, K]
        gap = np.where(np.isfinite(su[:, K]), gap, np.inf)
    else:
        gap = np.full(u.shape[0], np.inf)
    return order, gap


def _pad_rows(rows: list[list[int]], width: int) -> np.ndarray:
    out = np.full((len(rows), max(width, 1)), -1, dtype=np.int64)
    for r, row in enumerate(rows):
        out[r, :len(row)] = row
    return out


def route(q: np.ndarray, k: np.ndarray, pyr: list[np.ndarray], ts: np.ndarray, K: int,
          C: int = 64, g: int = 2, scale: float | None = None, record: bool = False, score: str = "lse"):
    """Top-down hierarchical selection for a batch of query tokens [Core: eq. 16-21; Steps: eq. 22].

    q      [T, G, d]  the G query heads of one GQA group at each token (float64)
    k      [n, d]     raw keys of the group's KV head
    pyr    levels from ``build_pyramid`` (built over all n keys, R1)
    ts     [T]        query positions

    Starting from A^(L) = {root}: at each level with more than K candidates,
    score every candidate i by s_i = log sum_{r in Ch(i)} exp(q . k_bar_r *
    scale) over its valid children (raw keys at the leaf level), sum s over
    the group's heads (u_i, eq. 22), keep K by (u desc, index asc) and expand
    the survivors to their valid children.  At level 1 the survivors are I_t.
    ``score`` picks the candidate score: "lse" (the method), "mean" or "mean_var"
    (the PISA-1 / PISA-2 variants, R8).

    Returns ``sel`` [T, K] (ascending, -1 padded) and ``gap`` [T], the
    smallest K-th minus (K+1)-th score difference over the scored levels
    (inf if no level was scored).  With ``record`` also returns a dict with
    the leaf candidates, their u (NaN where unscored) and per-level
    candidate counts.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    ts = np.asarray(ts, dtype=np.int64)
    T, G, d = q.shape
    n = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = len(pyr)
    sizes = [lv.shape[0] for lv in pyr]
    cand = np.zeros((T, 1), dtype=np.int64)          # A^(L) = {root}
    gap = np.full(T, np.inf)
    counts = []
    leaf_u = None
    for lvl in range(L, 0, -1):
        valid_c = cand >= 0
        n_c = valid_c.sum(axis=1)
        counts.append(n_c.copy())
        need = n_c > K
        survivors = cand
        u = np.full(cand.shape, np.nan)
        if need.any():
            rows = np.nonzero(need)[0]
            cr = cand[rows]
            if lvl > 1:
                kids = cr[:, :, None] * g + np.arange(g)[None, None, :]            # [R, W, g]
                ok = (cr[:, :, None] >= 0) & (kids < sizes[lvl - 2]) & \
                     (first_token(lvl - 1, kids, C, g) <= ts[rows, None, None])
                vecs = pyr[lvl - 2][np.where(ok, kids, 0)]                         # [R, W, g, d]
            else:
                kids = cr[:, :, None] * C + np.arange(C)[None, None, :]            # [R, W, C]
                ok = (cr[:, :, None] >= 0) & (kids < n) & (kids <= ts[rows, None, None])
                vecs = k[np.where(ok, kids, 0)]                                    # [R, W, C, d]
            R, W, c = ok.shape
            z = np.matmul(vecs.reshape(R, W * c, d), np.transpose(q[rows], (0, 2, 1))) * scale
            z = np.transpose(z.reshape(R, W, c, G), (0, 3, 1, 2))                  # [R, G, W, c]
            s = child_score(z, ok[:, None, :, :], score)                           # [R, G, W]
            ur = s.sum(axis=1)                                                     # [R, W]
            ur = np.where(cr >= 0, ur, NEG_INF)
            order, gr = _select_k(ur, cr, K)
            gap[rows] = np.minimum(gap[rows], gr)
            kept = np.take_along_axis(cr, order[:, :K], axis=-1)
            survivors = np.full((T, K), -1, dtype=np.int64)
            keep_rows = np.nonzero(~need)[0]
            survivors[keep_rows, :min(K, cand.shape[1])] = cand[keep_rows, :K]
            survivors[rows] = kept
            u[rows] = np.where(cr >= 0, ur, np.nan)
        if lvl == 1:
            if record:
                leaf_u = u
            leaf_cand = cand
            final = survivors
            break
        # expand survivors to their valid children at level lvl-1
        kids = survivors[:, :, None] * g + np.arange(g)[None, None, :]
        ok = (survivors[:, :, None] >= 0) & (kids < sizes[lvl - 2]) & \
             (first_token(lvl - 1, kids, C, g) <= ts[:, None, None])
        rows = [sorted(int(x) for x in kids[r][ok[r]]) for r in range(T)]
        cand = _pad_rows(rows, max((len(r) for r in rows), default=1))
    sel = np.full((T, K), -1, dtype=np.int64)
    for r in range(T):
        chosen = sorted(int(x) for x in final[r] if x >= 0)
        sel[r, :len(chosen)] = chosen
    if record:
        return sel, gap, {"leaf_cand": leaf_cand, "leaf_u": leaf_u, "counts": counts[::-1]}
    return sel, gap


def flat_mean_select(q: np.ndarray, leaves: np.ndarray, ts: np.ndarray, K: int, C: int = 64,
                     scale: float | None = None, return_scores: bool = False):
    """Single-level block selection of the block-sparse framework [Prereq/BSA; R7].

    q       [T, G, d]  the group's query heads at each token (float64)
    leaves  [M_1, d]   leaf means (level 1 of ``build_pyramid``)
    ts      [T]        query positions

    Every leaf j with j * C <= t is scored by u_j = sum over heads of
    q_h . k_bar_j * scale; K are kept by (u desc, j asc) [R3].  Returns ``sel``
    [T, K] (ascending, -1 padded) and ``gap`` [T] (K-th minus (K+1)-th score, inf
    when at most K leaves are valid); with ``return_scores`` also the scores of
    the selected leaves in ``sel`` order (-inf on padding).
    """
    q = np.asarray(q, dtype=np.float64)
    leaves = np.asarray(leaves, dtype=np.float64)
    ts = np.asarray(ts, dtype=np.int64)
    T, G, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    M = leaves.shape[0]
    z = np.einsum("tgd,md->tgm", q, leaves) * scale                   # [T, G, M]
    u = z.sum(axis=1)                                                   # [T, M]
    ids = np.broadcast_to(np.arange(M), (T, M))
    valid = ids * C <= ts[:, None]
    u = np.where(valid, u, NEG_INF)
    ids = np.where(valid, ids, -1)
    order, gap = _select_k(u, ids, K)
    top_ids = np.take_along_axis(ids, order[:, :K], axis=-1)
    top_u = np.take_along_axis(u, order[:, :K], axis=-1)
    sel = np.full((T, K), -1, dtype=np.int64)
    sel_u = np.full((T, K), NEG_INF)
    for r in range(T):
        keep = top_ids[r] >= 0
        pairs = sorted(zip(top_ids[r][keep].tolist(), top_u[r][keep].tolist()))
        sel[r, :len(pairs)] = [j for j, _ in pairs]
        sel_u[r, :len(pairs)] = [v for _, v in pairs]
    return (sel, gap, sel_u) if return_scores else (sel, gap)


def leaf_lse(q: np.ndarray, k: np.ndarray, j: int, t: int, C: int = 64,
             scale: float | None = None) -> np.ndarray:
    """Per-head exact LSE of query t over the raw keys of leaf j at positions <= t [Prereq/LSE; Core: eq. 21 at l = 1]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    keys = np.asarray(k, dtype=np.float64)[j * C:min((j + 1) * C, t + 1, k.shape[0])]
    return logsumexp(q @ keys.T * scale, axis=-1)


# ----------------------------------------------------------------------------- attention
def union_rows(sel: np.ndarray) -> np.ndarray:
    """Each row's listed block ids as a set (R5): repeats become -1 (int64, same shape)."""
    srt = np.sort(np.asarray(sel, dtype=np.int64), axis=1)
    repeat = np.zeros(srt.shape, dtype=bool)
    repeat[:, 1:] = srt[:, 1:] == srt[:, :-1]
    return np.where(repeat, -1, srt)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, ts: np.ndarray,
              C: int = 64, scale: float | None = None):
    """Softmax attention of each token's group heads over its selected blocks [Prereq/BSA; Steps: fourth step].

    Keys are the union of blocks j in I_t, positions [jC, min((j+1)C, n))
    cut to <= t (R5): a block listed twice contributes its keys once, and
    entries < 0 or past t contribute none.  Returns (o [T, G, d], lse [T, G],
    weight sums [T, G]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    ts = np.asarray(ts, dtype=np.int64)
    T, G, d = q.shape
    n = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    sel = union_rows(sel)
    Ks = sel.shape[1]
    pos = sel[:, :, None] * C + np.arange(C)[None, None, :]
    ok = (sel[:, :, None] >= 0) & (pos < n) & (pos <= ts[:, None, None])
    pos = np.where(ok, pos, 0).reshape(T, Ks * C)
    ok = ok.reshape(T, Ks * C)
    logits = np.matmul(q, np.transpose(k[pos], (0, 2, 1))) * scale                 # [T, G, Ks*C]
    logits = np.where(ok[:, None, :], logits, NEG_INF)
    lse = logsumexp(logits, axis=-1)
    p = np.exp(logits - lse[..., None])
    o = np.matmul(p, v[pos])                                                      # [T, G, d]
    return o, lse, p.sum(axis=-1)


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, ts: np.ndarray,
                       do: np.ndarray, C: int = 64, scale: float | None = None):
    """Gradients of `attention` for one (b, kvh) slice with the selections held fixed (R9).

    For each token t and head h with logits s = scale q . k_r over the keys r of its
    selected blocks (cut to r <= t), P = softmax(s), O = P V and upstream gradient dO:
      dV_r += P_r dO,   dP_r = dO . v_r,   Delta = sum_r P_r dP_r (= dO . O),
      dS_r = P_r (dP_r - Delta),   dq = scale sum_r dS_r k_r,   dk_r += scale dS_r q.
    Tokens are the rows ts of q / do; keys that several tokens select collect every
    token's contribution.  Returns (dq [T, G, d], dk [n, d], dv [n, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    ts = np.asarray(ts, dtype=np.int64)
    T, G, d = q.shape
    n = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(T):
        t = int(ts[r])
        blocks = sorted({int(j) for j in sel[r] if j >= 0})         # the union of the listed blocks (R5)
        pos = np.array([p for j in blocks for p in range(j * C, min((j + 1) * C, n)) if p <= t], dtype=np.int64)
        if pos.size == 0:
            continue
        kr, vr = k[pos], v[pos]                                     # [m, d]
        s = (q[r] @ kr.T) * scale                                   # [G, m]
        p = np.exp(s - logsumexp(s, axis=-1)[:, None])
        dp = do[r] @ vr.T                                           # [G, m]
        delta = (p * dp).sum(axis=-1, keepdims=True)
        ds = p * (dp - delta)
        dq[r] = scale * (ds @ kr)
        np.add.at(dk, pos, scale * (ds.T @ q[r]))
        np.add.at(dv, pos, p.T @ do[r])
    return dq, dk, dv


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, ts: np.ndarray,
                           scale: float | None = None) -> np.ndarray:
    """Textbook causal softmax attention over keys [0, t] (no selection)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    out = np.empty_like(q)
    for r, t in enumerate(np.asarray(ts)):
        a = q[r] @ k[:t + 1].T * scale
        a = np.exp(a - a.max(axis=-1, keepdims=True))
        out[r] = (a / a.sum(axis=-1, keepdims=True)) @ v[:t + 1]
    return out


# ----------------------------------------------------------------------------- whole prefill / decode
def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, K: int, C: int = 64, g: int = 2,
            ts=None, scale: float | None = None, chunk: int = 32, score: str = "lse"):
    """Selection and attention for one (sequence, KV head): q [n, G, d], k/v [n, d].

    ``ts`` restricts the queries evaluated (default: all n).  Returns a dict
    with ``sel`` [T, K], ``gap`` [T], ``o`` [T, G, d], ``lse`` [T, G].
    """
    n = k.shape[0]
    ts = np.arange(n) if ts is None else np.asarray(ts, dtype=np.int64)
    pyr = build_pyramid(k, C, g)
    sels, gaps, outs, lses = [], [], [], []
    for s in range(0, len(ts), chunk):
        tc = ts[s:s + chunk]
        sel, gap = route(q[tc], k, pyr, tc, K, C, g, scale, score=score)
        o, lse, _ = attention(q[tc], k, v, sel, tc, C, scale)
        sels.append(sel); gaps.append(gap); outs.append(o); lses.append(lse)
    return {"sel": np.concatenate(sels), "gap": np.concatenate(gaps),
            "o": np.concatenate(outs), "lse": np.concatenate(lses), "ts": ts}


class DecodeState:
    """KV cache and pyramid of one (sequence, KV head) for the decode oracle [Steps: third step].

    The cache is preallocated for ``capacity`` keys; ``n`` keys are present.
    """

    def __init__(self, k: np.ndarray, v: np.ndarray, C: int = 64, g: int = 2, capacity: int | None = None):
        n, d = k.shape
        capacity = n + 1024 if capacity is None else capacity
        self.kbuf = np.zeros((capacity, d))
        self.vbuf = np.zeros((capacity, d))
        self.kbuf[:n] = k
        self.vbuf[:n] = v
        self.C, self.g = C, g
        self.n = n
        self.pyr = build_pyramid(self.kbuf[:n], C, g) if n else []

    def keys(self) -> np.ndarray:
        return self.kbuf[:self.n]

    def values(self) -> np.ndarray:
        return self.vbuf[:self.n]

    def step(self, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, K: int,
             scale: float | None = None, score: str = "lse"):
        """Append (k_new, v_new) at position n, update the pyramid, route q at t = n, attend (R6)."""
        self.kbuf[self.n] = k_new
        self.vbuf[self.n] = v_new
        self.n += 1
        keys = self.keys()
        self.pyr = update_pyramid(self.pyr, keys, self.n, self.C, self.g)
        t = np.array([self.n - 1])
        qq = np.asarray(q, dtype=np.float64)[None]
        sel, gap = route(qq, keys, self.pyr, t, K, self.C, self.g, scale, score=score)
        o, lse, _ = attention(qq, keys, self.values(), sel, t, self.C, scale)
        return sel[0], gap[0], o[0], lse[0]
