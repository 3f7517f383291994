"""Second, independently written statement of PISA selection, for pinning the main oracle.

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over one query at a time,
meant for tiny inputs.  It shares no code with ``oracle.pisa``: it builds
its own pyramid by recursion over spans, computes LogSumExp with
``math.fsum`` (or exactly, with ``decimal`` at 50 digits), and orders
candidates with ``sorted``.

Rules follow the paper-summary page "Block Sparse Attention with Log-Linear
Complexity": pyramid means (Method steps, first step), LSE score over
children (Core method, eq. 21), group head sum (Method steps, eq. 22),
bounded top-down routing (Core method, eq. 16-20), and the same readings
for silent points as the main oracle (unweighted partial nodes, causal
validity by first token, ties to the lower index, no forced blocks).
"""
from __future__ import annotations

import decimal
import math


def _mean(vectors):
    d = len(vectors[0])
    return [math.fsum(vec[c] for vec in vectors) / len(vectors) for c in range(d)]


class Pyramid:
    """Recursive mean-pooled pyramid: node(level, i) is computed on demand and memoised."""

    def __init__(self, keys, C, g):
        self.keys = [list(map(float, row)) for row in keys]
        self.C, self.g = C, g
        self.sizes = {}
        m = -(-len(self.keys) // C)
        level = 1
        self.sizes[level] = m
        while m > 1:
            m = -(-m // g)
            level += 1
            self.sizes[level] = m
        self.top = level
        self._memo = {}

    def children(self, level, i):
        """Children indices of node (level, i) one level down (raw key positions for level 1)."""
        if level == 1:
            return list(range(i * self.C, min((i + 1) * self.C, len(self.keys))))
        return [c for c in range(i * self.g, i * self.g + self.g) if c < self.sizes[level - 1]]

    def first(self, level, i):
        return i * self.C * self.g ** (level - 1)

    def vector(self, level, i):
        if level == 0:
            return self.keys[i]
        key = (level, i)
        if key not in self._memo:
            self._memo[key] = _mean([self.vector(level - 1, c) for c in self.children(level, i)])
        return self._memo[key]


def dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def lse(values):
    m = max(values)
    return m + math.log(math.fsum(math.exp(v - m) for v in values))


def lse_exact(values, digits: int = 50):
    """LogSumExp with 50-digit decimal arithmetic from the exact binary inputs."""
    with decimal.localcontext() as ctx:
        ctx.prec = digits
        total = sum(decimal.Decimal(v).exp() for v in values)
        return float(total.ln())


def _reduce(values, mode):
    """LSE, or the mean / mean + half population variance of the score variants."""
    if mode == "lse":
        return lse(values)
    mean = math.fsum(values) / len(values)
    if mode == "mean":
        return mean
    return mean + 0.5 * math.fsum((v - mean) ** 2 for v in values) / len(values)


def score(pyr: Pyramid, heads, level, i, t, scale, mode="lse"):
    """u = sum over heads of the score (LSE, or a variant) over the valid children of node (level, i)."""
    kids = pyr.children(level, i)
    if level == 1:
        kids = [r for r in kids if r <= t]
    else:
        kids = [c for c in kids if pyr.first(level - 1, c) <= t]
    return math.fsum(_reduce([dot(q, pyr.vector(level - 1, c)) * scale for c in kids], mode) for q in heads)


def select(keys, heads, t, K, C=64, g=2, scale=None, pyr=None, mode="lse", with_gap=False):
    """Leaf block ids chosen for query position t (sorted ascending).

    With ``with_gap`` also returns the boundary margin of the acceptance rule:
    at every level holding more than K candidates, the K-th largest score
    minus the (K+1)-th, and the smallest of these over the levels (inf when no
    level was scored).
    """
    pyr = pyr or Pyramid(keys, C, g)
    scale = 1.0 / math.sqrt(len(heads[0])) if scale is None else scale
    level = pyr.top
    cand = [0]
    margins = []
    while True:
        if len(cand) > K:
            scored = {i: score(pyr, heads, level, i, t, scale, mode) for i in cand}
            ranked = sorted(cand, key=lambda i: (-scored[i], i))
            margins.append(scored[ranked[K - 1]] - scored[ranked[K]])
            cand = ranked[:K]
        if level == 1:
            if with_gap:
                return sorted(cand), min(margins, default=math.inf)
            return sorted(cand)
        nxt = []
        for i in cand:
            nxt += [c for c in pyr.children(level, i) if pyr.first(level - 1, c) <= t]
        cand = nxt
        level -= 1


def flat_select(keys, heads, t, K, C=64, scale=None):
    """Brute force: exact leaf LSE of every causally valid leaf, summed over heads, top K."""
    scale = 1.0 / math.sqrt(len(heads[0])) if scale is None else scale
    n = len(keys)
    scores = []
    for j in range(-(-n // C)):
        if j * C > t:
            break
        block = [keys[r] for r in range(j * C, min((j + 1) * C, n)) if r <= t]
        u = math.fsum(lse([dot(q, key) * scale for key in block]) for q in heads)
        scores.append((-u, j))
    return sorted(j for _, j in sorted(scores)[:K])


def attend(keys, values, heads, blocks, t, C=64, scale=None):
    """Softmax attention of each head over the keys of ``blocks`` at positions <= t (a block
    listed twice counts once)."""
    scale = 1.0 / math.sqrt(len(heads[0])) if scale is None else scale
    pos = [r for j in sorted(set(blocks)) if j >= 0 for r in range(j * C, min((j + 1) * C, len(keys))) if r <= t]
    out = []
    for q in heads:
        logits = [dot(q, keys[r]) * scale for r in pos]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        z = math.fsum(w)
        out.append([math.fsum(w[a] * values[r][c] for a, r in enumerate(pos)) / z
                    for c in range(len(values[0]))])
    return out
