"""The routing pre-filter's per-logit bound, checked on the host (no GPU).

The bf16 routing pre-filter (route.hip) scores a child from a float16 copy x16 of its float32
summary x and bounds the distance to the score from the split parts (hi = bf16(x) and
lo = f16((x - hi) 2^10)) by |q| R + |q - q_lo| X (1 + 2^-15) + 2^-24 |y|, with the per-node R and X
that split_summaries_kernel forms.  Here the same quantities are formed independently with NumPy,
rounding emulated exactly (bf16 to nearest even on float32 bits, float16 through NumPy, float32
sums of the exact products in several orders, one of them truncating every addition), and the
distance between the two float32 logits is checked against the bound for random and adversarial
rows: overflowing and subnormal float16 values, mixed scales, exact bf16 values, and queries with
elements outside the float16 normal range.
"""
from __future__ import annotations

import numpy as np
import pytest

F32 = np.float32


def bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest even), returned as float32 values."""
    b = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(F32)


def f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16 after clamping to the float16 range, returned as float32 values."""
    return np.clip(x, -65504.0, 65504.0).astype(np.float16).astype(F32)


def trunc_add(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """float32 addition rounded toward zero."""
    exact = a.astype(np.float64) + b.astype(np.float64)
    r = exact.astype(F32)
    over = np.abs(r.astype(np.float64)) > np.abs(exact)
    return np.where(over, np.nextafter(r, F32(0)), r)


def sums(p: np.ndarray, rng) -> list[np.ndarray]:
    """float32 sums over the last axis of exact float32 products, in several orders."""
    out = []
    s = np.zeros(p.shape[:-1], F32)
    for i in range(p.shape[-1]):                       # in order
        s = F32(s + p[..., i])
    out.append(s)
    t = np.zeros(p.shape[:-1], F32)
    for i in reversed(range(p.shape[-1])):             # reversed, truncating
        t = trunc_add(t, p[..., i])
    out.append(t)
    blocks = p.reshape(p.shape[:-1] + (-1, 32))        # 32-product steps, pairwise inside each
    v = blocks
    while v.shape[-1] > 1:
        v = F32(v[..., 0::2] + v[..., 1::2])
    c = np.zeros(p.shape[:-1], F32)
    for j in range(v.shape[-2]):
        c = F32(c + v[..., j, 0])
    out.append(c)
    perm = rng.permutation(p.shape[-1])                # a random order
    r = np.zeros(p.shape[:-1], F32)
    for i in perm:
        r = F32(r + p[..., i])
    out.append(r)
    return out


def node_bounds(x: np.ndarray):
    """R and X of each row as split_summaries_kernel forms them (here in float64, then rounded up
    the way the kernel does), with the split parts and the float16 copy."""
    hi = bf16(x)
    lo = f16(F32(x - hi) * F32(1024.0))
    x16 = f16(x)
    lo_s = lo.astype(np.float64) * 2.0 ** -10
    rho = (x.astype(np.float64) - hi) - lo_s
    xi = x.astype(np.float64) - x16
    nrm = lambda v: np.sqrt(np.sum(np.square(v.astype(np.float64)), axis=-1))
    R = (nrm(rho) + nrm(xi)) * 1.0000306 + 2.0 ** -15 * 1.01 * (nrm(hi) + nrm(lo_s) + nrm(x16)) + 2.0 ** -60
    X = (nrm(lo_s) + nrm(x16)) * 1.0000306 + 2.0 ** -60
    return hi, lo, x16, R, X


def check(q: np.ndarray, x: np.ndarray, rng):
    """q [d] bf16 values, x [rows, d] float32 summaries."""
    q = bf16(q)
    q_lo = f16(q)
    hi, lo, x16, R, X = node_bounds(x)
    qn = np.sqrt(np.sum(q.astype(np.float64) ** 2))
    qd = np.sqrt(np.sum((q.astype(np.float64) - q_lo) ** 2))
    p_hi = F32(q * hi)                                 # products of bf16 values: exact in float32
    p_lo = F32(q_lo * lo)                              # products of float16 values: exact
    p_16 = F32(q_lo * x16)
    worst = 0.0
    for s_hi in sums(p_hi, rng):
        for s_lo in sums(p_lo, rng):
            y_split = F32(s_hi + F32(s_lo * F32(2.0 ** -10)))
            for y16 in sums(p_16, rng):
                bound = (qn * R + qd * X * 1.0001 + 2.0 ** -24 * np.abs(y16.astype(np.float64))) * 1.0001 + 2.0 ** -40
                dist = np.abs(y_split.astype(np.float64) - y16.astype(np.float64))
                assert np.all(dist <= bound), (float(np.max(dist - bound)),)
                worst = max(worst, float(np.max(dist / bound)))
    return worst


@pytest.mark.parametrize("d", [64, 128])
def test_bound_holds_on_normal_rows(d):
    rng = np.random.default_rng(d)
    q = rng.standard_normal(d).astype(F32)
    for scale in (1.0, 1 / 8, 1 / 64, 1 / 512):        # leaf means and coarser summaries shrink
        x = (rng.standard_normal((256, d)) * scale).astype(F32)
        worst = check(q, x, rng)
        assert worst < 1.0


def test_bound_holds_on_adversarial_rows():
    rng = np.random.default_rng(7)
    d = 128
    q = rng.standard_normal(d).astype(F32)
    rows = [
        rng.standard_normal((64, d)) * 1e6,            # beyond the float16 range: x16 clamped
        rng.choice([-1.0, 1.0], (64, d)) * rng.uniform(33000, 65000, (64, d)),   # x16 in range, lo clamped
        rng.standard_normal((64, d)) * 1e-6,           # float16 subnormal copies
        rng.standard_normal((64, d)) * 1e-12,          # below every float16
        rng.standard_normal((64, d)) * np.where(rng.random((64, d)) < 0.5, 1e4, 1e-5),   # mixed scales
        bf16(rng.standard_normal((64, d)).astype(F32)),   # exact bf16 values: lo = 0
        np.full((64, d), 0.375),
    ]
    for x in rows:
        check(q, np.asarray(x, dtype=F32), rng)
    # a query aligned with a clamped remainder: 40100 rounds to the bf16 value 40192, the remainder
    # -92 leaves the float16 range after the 2^10 scaling (rho = -28), while f16 holds 40096 (xi = 4)
    check(np.full(d, -1.0, F32), np.full((4, d), 40100.0, F32), rng)
    # queries with elements below the float16 normal range or beyond its largest value
    x = rng.standard_normal((64, d)).astype(F32) / 8
    q_sub = np.where(rng.random(d) < 0.2, q * 1e-6, q).astype(F32)
    check(q_sub, x, rng)
    q_big = q.copy()
    q_big[:3] = 1e6
    check(q_big, x, rng)


def test_bound_is_tight_enough_to_help():
    """For N(0,1) queries and leaf-mean-sized rows the bound is far below the spread of the logits,
    which is what lets most candidates be decided without the split rows."""
    rng = np.random.default_rng(11)
    d = 128
    q = bf16(rng.standard_normal(d).astype(F32))
    x = (rng.standard_normal((512, d)) / 8).astype(F32)
    _, _, _, R, X = node_bounds(x)
    bound = np.sqrt(np.sum(q.astype(np.float64) ** 2)) * R
    spread = np.std(x.astype(np.float64) @ q.astype(np.float64))
    assert np.median(bound) < 1e-2 * spread          # about 0.3% here
