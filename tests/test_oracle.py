"""Pins for the CPU oracle: closed forms, brute force, hand-derived fixtures and invariants.

Everything here runs on the CPU in seconds.  Each test states which rule of
the paper-summary page "Block Sparse Attention with Log-Linear Complexity"
it pins, and checks the oracle against something other than itself.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import per_query
from oracle import pisa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- pyramid
def test_pyramid_full_spans_equal_span_means():
    """Method steps, first step: with n = C * g**(L-1) every node is the mean of its key span."""
    C, g = 4, 2
    k = _rand(1, 64, 3)
    pyr = pisa.build_pyramid(k, C, g)
    assert [lv.shape[0] for lv in pyr] == [16, 8, 4, 2, 1]
    for lvl, nodes in enumerate(pyr, start=1):
        span = C * g ** (lvl - 1)
        for i in range(nodes.shape[0]):
            np.testing.assert_allclose(nodes[i], k[i * span:(i + 1) * span].mean(axis=0), rtol=0, atol=1e-14)


def test_pyramid_partial_nodes_golden():
    """Partial nodes are the unweighted mean of existing children (hand-derived fixture)."""
    with open(os.path.join(GOLDEN, "pyramid_partial.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        pyr = pisa.build_pyramid(np.array(case["keys"], dtype=float), C=2, g=2)
        assert len(pyr) == len(case["levels"])
        for got, want in zip(pyr, case["levels"]):
            np.testing.assert_array_equal(got, np.array(want, dtype=float))


def test_pyramid_invariant_to_key_order_within_span():
    C, g = 8, 2
    k = _rand(2, 64, 4)
    perm = k.copy()
    perm[8:16] = perm[8:16][::-1]
    a, b = pisa.build_pyramid(k, C, g), pisa.build_pyramid(perm, C, g)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-14)


@pytest.mark.parametrize("C", [1, 2, 4])
def test_incremental_update_equals_rebuild(C):
    """Method steps, third step: updating the new leaf and its ancestors equals a rebuild."""
    k = _rand(3, 70, 3)
    pyr = pisa.build_pyramid(k[:1], C, 2)
    for n in range(2, 71):
        pyr = pisa.update_pyramid(pyr, k, n, C, 2)
        ref = pisa.build_pyramid(k[:n], C, 2)
        assert len(pyr) == len(ref), n
        for x, y in zip(pyr, ref):
            np.testing.assert_array_equal(x, y)


def test_level_sizes():
    assert pisa.level_sizes(1024, 64, 2) == [16, 8, 4, 2, 1]
    assert pisa.level_sizes(262144, 64, 2)[0] == 4096 and len(pisa.level_sizes(262144)) == 13
    assert pisa.level_sizes(131073, 64, 2)[:2] == [2049, 1025] and len(pisa.level_sizes(131073)) == 13
    assert len(pisa.level_sizes(131072)) == 12


# ----------------------------------------------------------------------------- LSE
def test_logsumexp_matches_50_digit_decimal():
    """Prerequisites, LogSumExp: log sum exp z, checked against 50-digit arithmetic."""
    rng = np.random.default_rng(4)
    for scale in (1e-3, 1.0, 30.0, 300.0):
        z = rng.standard_normal(64) * scale
        assert abs(pisa.logsumexp(z) - per_query.lse_exact(list(z))) <= 1e-13 * max(1.0, abs(per_query.lse_exact(list(z))))


def test_logsumexp_bounds_and_identical_entries():
    """Prerequisites, LogSumExp: smooth upper bound of max; m equal entries give z + log m."""
    rng = np.random.default_rng(5)
    for m in (1, 2, 7, 64):
        z = rng.standard_normal(m) * 3
        s = pisa.logsumexp(z)
        assert z.max() <= s <= z.max() + math.log(m) + 1e-12
        assert abs(pisa.logsumexp(np.full(m, 0.37)) - (0.37 + math.log(m))) < 1e-14


def test_logsumexp_taylor_expansion():
    """Core method: LSE = log m + mean + Var/2 + O(eps^3) for logits of size eps."""
    x = np.random.default_rng(6).standard_normal(64)
    res = []
    for eps in (1e-1, 5e-2, 2.5e-2):
        z = eps * x
        res.append(abs(pisa.logsumexp(z) - (math.log(64) + z.mean() + 0.5 * z.var())))
    assert 5.0 < res[0] / res[1] < 11.0 and 5.0 < res[1] / res[2] < 11.0   # cubic: ratio ~8


def test_leaf_lse_exact_and_causal():
    """Core method eq. 21 at the leaf level: exact LSE over the block's raw keys at positions <= t."""
    q = _rand(7, 3, 8)
    k = _rand(8, 40, 8)
    scale = 1 / math.sqrt(8)
    for j, t in [(0, 39), (1, 25), (2, 33), (1, 16)]:
        got = pisa.leaf_lse(q, k, j, t, C=16)
        keys = [k[r] for r in range(j * 16, min((j + 1) * 16, 40)) if r <= t]
        want = [per_query.lse_exact([float(np.dot(qh, kk)) * scale for kk in keys]) for qh in q]
        np.testing.assert_allclose(got, want, rtol=1e-13)


# ----------------------------------------------------------------------------- routing
def test_route_golden_hand_examples():
    """Hand-derived routing examples with a deliberate difference from flat top-1 and an exact tie."""
    with open(os.path.join(GOLDEN, "route_tiny.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        K = case.get("K", 1)
        k = np.array(case["keys"], dtype=float)[:, None]
        pyr = pisa.build_pyramid(k, C=1, g=2)
        sel, _ = pisa.route(np.ones((1, 1, 1)), k, pyr, np.array([case["t"]]), K=K, C=1, g=2, scale=1.0)
        assert [int(x) for x in sel[0] if x >= 0] == case["expected"], case
        heads = [[1.0]]
        assert per_query.select([[x] for x in case["keys"]], heads, case["t"], K, C=1, g=2, scale=1.0) == case["expected"]


def test_route_boundary_gap_golden():
    """The acceptance rule's boundary record (K-th minus (K+1)-th score, smallest over the scored
    levels) against hand-derived values: cases where the minimum sits at an upper level, at the
    leaf level and at a middle level, and where the neighbouring differences of the sorted scores
    (an off-by-one in the positions) or the largest level margin would give another number."""
    with open(os.path.join(GOLDEN, "route_tiny.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        K = case.get("K", 1)
        assert case["gap"] == min(case["level_gaps"])
        k = np.array(case["keys"], dtype=float)[:, None]
        pyr = pisa.build_pyramid(k, C=1, g=2)
        _, gap = pisa.route(np.ones((1, 1, 1)), k, pyr, np.array([case["t"]]), K=K, C=1, g=2, scale=1.0)
        assert abs(gap[0] - case["gap"]) <= 1e-6, (case["keys"], case["t"], gap[0], case["gap"])
        sel, pq_gap = per_query.select([[x] for x in case["keys"]], [[1.0]], case["t"], K, C=1, g=2, scale=1.0,
                                       with_gap=True)
        assert sel == case["expected"] and abs(pq_gap - case["gap"]) <= 1e-6, (case["keys"], pq_gap)


@pytest.mark.parametrize("seed", range(4))
def test_route_gap_agrees_with_independent_per_query_routine(seed):
    """The boundary record of the level-wise oracle equals the independently written per-query
    routine's (its own pyramid, LSE and sort) on random tiny inputs, ties included."""
    rng = np.random.default_rng(300 + seed)
    C, G, K, n = [(2, 2, 2, 60), (4, 1, 3, 100), (4, 3, 2, 90), (2, 2, 4, 70)][seed]
    k = np.round(rng.standard_normal((n, 4)) * 2) / 2         # coarse values: some exact ties
    q = np.round(rng.standard_normal((n, G, 4)) * 2) / 2 + 0.5
    pyr = pisa.build_pyramid(k, C, 2)
    sel, gap = pisa.route(q, k, pyr, np.arange(n), K, C, 2)
    ref_pyr = per_query.Pyramid(k.tolist(), C, 2)
    n_zero = n_inf = 0
    for t in range(n):
        want, want_gap = per_query.select(k.tolist(), q[t].tolist(), t, K, C, 2, pyr=ref_pyr, with_gap=True)
        assert [int(x) for x in sel[t] if x >= 0] == want, t
        if math.isinf(want_gap):
            assert math.isinf(gap[t]), (t, gap[t])
            n_inf += 1
        else:
            assert abs(gap[t] - want_gap) <= 1e-9 * max(1.0, abs(want_gap)), (t, gap[t], want_gap)
            n_zero += want_gap == 0.0
    assert n_inf > 0 and n_inf < n                             # early tokens score no level


@pytest.mark.parametrize("C,G,n", [(4, 1, 40), (4, 2, 64), (8, 4, 72), (2, 3, 33)])
def test_flat_equivalence_when_every_level_is_kept(C, G, n):
    """Core method: when K >= ceil(M1/2), no level above the leaves is cut, so the result is the
    brute-force flat top-K over exact leaf LSE (summed over heads) of all valid leaves."""
    rng = np.random.default_rng(10 + C + G + n)
    k = rng.standard_normal((n, 6))
    q = rng.standard_normal((n, G, 6)) + 0.5
    m1 = -(-n // C)
    K = -(-m1 // 2)
    pyr = pisa.build_pyramid(k, C, 2)
    sel, _ = pisa.route(q, k, pyr, np.arange(n), K, C, 2)
    for t in range(n):
        want = per_query.flat_select(k.tolist(), q[t].tolist(), t, K, C)
        assert [int(x) for x in sel[t] if x >= 0] == want, t


@pytest.mark.parametrize("seed", range(6))
def test_route_agrees_with_independent_per_query_routine(seed):
    """General hierarchical case (K < ceil(M1/2)): two independently written routines agree."""
    rng = np.random.default_rng(100 + seed)
    C = [2, 4, 4, 8, 2, 4][seed]
    G = [1, 2, 4, 2, 3, 1][seed]
    K = [2, 2, 3, 2, 3, 4][seed]
    n = [50, 96, 128, 130, 77, 200][seed]
    k = rng.standard_normal((n, 5))
    k[C * 3:C * 4] += 1.5                         # one planted block
    q = rng.standard_normal((n, G, 5)) + 0.3
    pyr = pisa.build_pyramid(k, C, 2)
    sel, gap = pisa.route(q, k, pyr, np.arange(n), K, C, 2)
    ref_pyr = per_query.Pyramid(k.tolist(), C, 2)
    for t in range(n):
        want = per_query.select(k.tolist(), q[t].tolist(), t, K, C, 2, pyr=ref_pyr)
        assert [int(x) for x in sel[t] if x >= 0] == want, (t, gap[t])


def test_selection_size_validity_and_candidate_bound():
    """|I_t| = min(K, floor(t/C)+1), distinct, ascending, causally valid; at most gK candidates per level."""
    rng = np.random.default_rng(11)
    C, g, K, n = 4, 2, 3, 150
    k = rng.standard_normal((n, 4))
    q = rng.standard_normal((n, 2, 4))
    pyr = pisa.build_pyramid(k, C, g)
    sel, gap, rec = pisa.route(q, k, pyr, np.arange(n), K, C, g, record=True)
    for t in range(n):
        s = [int(x) for x in sel[t] if x >= 0]
        assert len(s) == min(K, t // C + 1)
        assert s == sorted(set(s)) and all(j * C <= t for j in s)
        assert all(x == -1 for x in sel[t][len(s):])
    for counts in rec["counts"]:
        assert counts.max() <= g * K


def test_ties_go_to_the_lower_index():
    """Identical keys tie at every level: the K lowest leaves win (tie rule reading)."""
    C, g, K = 4, 2, 3
    n = C * 16
    k = np.tile(_rand(12, 1, 5), (n, 1))
    q = _rand(13, 1, 2, 5)
    pyr = pisa.build_pyramid(k, C, g)
    sel, gap = pisa.route(q, k, pyr, np.array([n - 1]), K, C, g)
    assert list(sel[0]) == [0, 1, 2] and gap[0] == 0.0
    # two identical blocks compete for one slot: the lower one wins
    k2 = _rand(14, 8, 5)
    k2[4:8] = k2[0:4]
    pyr2 = pisa.build_pyramid(k2, C, g)
    sel2, _ = pisa.route(_rand(15, 1, 1, 5), k2, pyr2, np.array([7]), 1, C, g)
    assert list(sel2[0]) == [0]


def test_head_sum_is_group_invariant_and_single_head_reduces():
    """Method steps eq. 22: u sums the group's head scores (order of heads does not matter)."""
    rng = np.random.default_rng(16)
    C, K, n = 4, 2, 96
    k = rng.standard_normal((n, 6))
    q = rng.standard_normal((n, 4, 6))
    pyr = pisa.build_pyramid(k, C, 2)
    a, _ = pisa.route(q, k, pyr, np.arange(n), K, C, 2)
    b, _ = pisa.route(q[:, ::-1], k, pyr, np.arange(n), K, C, 2)
    np.testing.assert_array_equal(a, b)
    one, _ = pisa.route(q[:, :1], k, pyr, np.arange(n), K, C, 2)
    for t in range(0, n, 7):
        assert [int(x) for x in one[t] if x >= 0] == per_query.select(k.tolist(), q[t, :1].tolist(), t, K, C, 2)


# ----------------------------------------------------------------------------- attention
def test_all_leaves_selected_gives_dense_causal_attention():
    """K >= M1: every valid leaf is kept and attention is textbook dense causal attention."""
    rng = np.random.default_rng(17)
    C, n, G = 8, 60, 2
    k, v = rng.standard_normal((n, 5)), rng.standard_normal((n, 5))
    q = rng.standard_normal((n, G, 5))
    out = pisa.prefill(q, k, v, K=8, C=C)
    for t in range(n):
        assert [int(x) for x in out["sel"][t] if x >= 0] == list(range(t // C + 1))
    np.testing.assert_allclose(out["o"], pisa.dense_causal_attention(q, k, v, np.arange(n)), atol=1e-12)


def test_attention_weights_sum_to_one_and_first_token():
    rng = np.random.default_rng(18)
    C, n = 4, 40
    k, v = rng.standard_normal((n, 3)), rng.standard_normal((n, 3))
    q = rng.standard_normal((n, 2, 3)) * 4
    pyr = pisa.build_pyramid(k, C)
    ts = np.arange(n)
    sel, _ = pisa.route(q, k, pyr, ts, 2, C)
    o, lse, wsum = pisa.attention(q, k, v, sel, ts, C)
    np.testing.assert_allclose(wsum, 1.0, atol=1e-13)
    np.testing.assert_allclose(o[0], np.tile(v[0], (2, 1)), atol=1e-15)


def test_attention_matches_per_query_routine():
    rng = np.random.default_rng(19)
    C, n = 4, 30
    k, v = rng.standard_normal((n, 3)), rng.standard_normal((n, 3))
    q = rng.standard_normal((n, 2, 3))
    sel = np.array([[0, 2, -1], [1, 3, 5]])
    ts = np.array([9, 23])
    o, _, _ = pisa.attention(q[ts], k, v, sel, ts, C)
    for r, t in enumerate(ts):
        want = per_query.attend(k.tolist(), v.tolist(), q[t].tolist(), [x for x in sel[r] if x >= 0], t, C)
        np.testing.assert_allclose(o[r], want, atol=1e-13)


def _messy_rows(n, C, K, rng):
    """Rows listing every block j <= t / C (some twice, in random order) plus ids past t, -1 and
    ids beyond the last block."""
    m1 = -(-n // C)
    sel = np.full((n, K), -1, dtype=np.int64)
    for t in range(n):
        ids = list(range(t // C + 1))
        ids += list(rng.choice(ids, size=min(2, len(ids)), replace=False))          # repeats
        ids += [t // C + 1, m1 + 3, 10 ** 6, -1]                                     # past t / absent
        ids = list(rng.permutation(ids))
        sel[t, :len(ids)] = ids
    return sel


def test_attention_union_reading_reduces_to_dense_causal_attention():
    """Reading R5: the key set is the union of the listed blocks cut to <= t.  Rows that list every
    valid block, some of them twice and in random order, plus ids past t or past the last block,
    give textbook dense causal attention; the gradients equal float64 autograd of it."""
    import torch

    rng = np.random.default_rng(23)
    C, n, G, d = 8, 45, 2, 4
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    q = rng.standard_normal((n, G, d))
    do = rng.standard_normal((n, G, d))
    ts = np.arange(n)
    sel = _messy_rows(n, C, 16, rng)
    o, lse, wsum = pisa.attention(q, k, v, sel, ts, C)
    np.testing.assert_allclose(o, pisa.dense_causal_attention(q, k, v, ts), atol=1e-12)
    np.testing.assert_allclose(wsum, 1.0, atol=1e-13)
    for t in (0, 17, 44):                                        # the independent routine, same rows
        want = per_query.attend(k.tolist(), v.tolist(), q[t].tolist(), [int(x) for x in sel[t]], t, C)
        np.testing.assert_allclose(o[t], want, atol=1e-13)
    dq, dk, dv = pisa.attention_backward(q, k, v, sel, ts, do, C=C)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    logits = torch.einsum("tgd,sd->tgs", qt, kt) / math.sqrt(d)
    mask = torch.arange(n)[None, :] > torch.arange(n)[:, None]
    out = torch.einsum("tgs,sd->tgd", torch.softmax(logits.masked_fill(mask[:, None, :], float("-inf")), -1), vt)
    out.backward(torch.tensor(do))
    for got, want in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- decode
def test_decode_step_equals_prefill_of_last_token():
    """Method steps, third step: decode at length n+1 equals prefill's result for token n."""
    rng = np.random.default_rng(20)
    C, K, G, d = 4, 2, 2, 5
    n0, steps = 29, 40                 # crosses 32 and 64 keys: new leaves and a new root level
    k = rng.standard_normal((n0 + steps, d))
    v = rng.standard_normal((n0 + steps, d))
    q = rng.standard_normal((n0 + steps, G, d))
    st = pisa.DecodeState(k[:n0], v[:n0], C)
    for s in range(steps):
        n = n0 + s
        sel, gap, o, lse = st.step(q[n], k[n], v[n], K)
        ref_pyr = pisa.build_pyramid(k[:n + 1], C)
        assert len(st.pyr) == len(ref_pyr)
        for x, y in zip(st.pyr, ref_pyr):
            np.testing.assert_array_equal(x, y)
        want_sel, _ = pisa.route(q[n:n + 1], k[:n + 1], ref_pyr, np.array([n]), K, C)
        np.testing.assert_array_equal(sel, want_sel[0])
        want_o, _, _ = pisa.attention(q[n:n + 1], k[:n + 1], v[:n + 1], want_sel, np.array([n]), C)
        np.testing.assert_allclose(o, want_o[0], atol=1e-13)


# ----------------------------------------------------------------------------- flat (single-level) baseline
@pytest.mark.parametrize("C,G,m1", [(4, 1, 12), (4, 3, 16), (8, 2, 9)])
def test_flat_mean_equals_exact_lse_on_constant_key_blocks(C, G, m1):
    """Prerequisites (LSE paragraph): the LSE of m equal logits z is z + log m.  When every key of a
    block is the same vector, each full block's exact LSE is its mean score plus the same G log C,
    so the single-level mean selection must equal the independent brute-force exact-LSE flat top-K
    at every token that ends a block (all valid blocks full)."""
    rng = np.random.default_rng(300 + C + G + m1)
    d = 6
    block_keys = rng.standard_normal((m1, d))
    k = np.repeat(block_keys, C, axis=0)
    n = m1 * C
    q = rng.standard_normal((n, G, d)) + 0.4
    ts = np.arange(C - 1, n, C)
    leaves = pisa.build_pyramid(k, C, 2)[0]
    for K in (1, 3, m1):
        sel, gap = pisa.flat_mean_select(q[ts], leaves, ts, K, C)
        for r, t in enumerate(ts):
            want = per_query.flat_select(k.tolist(), q[t].tolist(), int(t), K, C)
            assert [int(x) for x in sel[r] if x >= 0] == want, (K, t, gap[r])


def test_flat_mean_is_the_small_logit_limit_of_exact_lse():
    """Prerequisites (LSE paragraph): log sum exp z = log m + mean(z) + Var(z)/2 + ..., so for tiny
    logits the exact-LSE ranking of full blocks follows the mean score (first-order term).  Checked
    against the independent brute force wherever the mean ranking's K-th gap dwarfs the variance term."""
    rng = np.random.default_rng(301)
    C, G, d, m1, K = 4, 2, 5, 20, 4
    k = rng.standard_normal((m1 * C, d))
    q = rng.standard_normal((m1 * C, G, d))
    scale = 1e-4
    ts = np.arange(C - 1, m1 * C, C)
    leaves = pisa.build_pyramid(k, C, 2)[0]
    sel, gap = pisa.flat_mean_select(q[ts], leaves, ts, K, C, scale)
    checked = 0
    for r, t in enumerate(ts):
        if gap[r] < 1e-6:                       # variance term is O(scale^2 |q|^2 |k|^2) ~ 1e-7
            continue
        want = per_query.flat_select(k.tolist(), q[t].tolist(), int(t), K, C, scale)
        assert [int(x) for x in sel[r] if x >= 0] == want, t
        checked += 1
    assert checked >= len(ts) // 2


def test_flat_mean_size_validity_planted_block_and_ties():
    """Selection-set invariants of the flat baseline: min(K, floor(t/C)+1) distinct ascending valid
    leaves; a strongly planted block is always kept once valid; duplicated blocks tie to the lower
    index (tie rule reading)."""
    rng = np.random.default_rng(302)
    C, G, d, n, K = 4, 2, 8, 120, 3
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    k = rng.standard_normal((n, d))
    k[5 * C:6 * C] += 6.0 * u                   # block 5
    q = rng.standard_normal((n, G, d)) + 4.0 * u
    ts = np.arange(n)
    leaves = pisa.build_pyramid(k, C, 2)[0]
    sel, gap = pisa.flat_mean_select(q, leaves, ts, K, C)
    for t in ts:
        s = [int(x) for x in sel[t] if x >= 0]
        assert len(s) == min(K, t // C + 1)
        assert s == sorted(set(s)) and all(j * C <= t for j in s)
        if t >= 5 * C:
            assert 5 in s
    k2 = rng.standard_normal((8 * C, d))
    k2[6 * C:7 * C] = k2[2 * C:3 * C]           # block 6 duplicates block 2
    leaves2 = pisa.build_pyramid(k2, C, 2)[0]
    qq = np.tile(leaves2[2], (1, 1, 1))         # the query points at block 2's mean: it ranks first
    sel2, gap2 = pisa.flat_mean_select(qq, leaves2, np.array([8 * C - 1]), 1, C)
    assert list(sel2[0]) == [2] and gap2[0] == 0.0


# ----------------------------------------------------------------------------- score variants (PISA-1, PISA-2)
@pytest.mark.parametrize("mode", ["mean", "mean_var"])
@pytest.mark.parametrize("seed", range(3))
def test_score_variants_agree_with_independent_per_query_routine(mode, seed):
    """The mean (PISA-1) and mean + var/2 (PISA-2) scores through the whole hierarchy: the vectorised
    oracle and the independently written per-query routine agree."""
    rng = np.random.default_rng(400 + seed)
    C, G, K, n = [(4, 2, 2, 96), (2, 3, 3, 77), (8, 1, 2, 130)][seed]
    k = rng.standard_normal((n, 5))
    k[C * 2:C * 3] += 1.2
    q = rng.standard_normal((n, G, 5)) + 0.3
    pyr = pisa.build_pyramid(k, C, 2)
    sel, gap = pisa.route(q, k, pyr, np.arange(n), K, C, 2, score=mode)
    ref_pyr = per_query.Pyramid(k.tolist(), C, 2)
    for t in range(n):
        want = per_query.select(k.tolist(), q[t].tolist(), t, K, C, 2, pyr=ref_pyr, mode=mode)
        assert [int(x) for x in sel[t] if x >= 0] == want, (t, gap[t])


def test_mean_var_score_is_the_second_order_truncation_of_lse():
    """Core method (Taylor expansion): LSE(z) = log m + mean + Var/2 + O(z^3).  The PISA-2 score must
    match LSE - log m with a residual shrinking like the cube of the logit scale, and the PISA-1
    score must match with a residual shrinking like its square (the variance term)."""
    rng = np.random.default_rng(401)
    z0 = rng.standard_normal((50, 7))
    ok = rng.random((50, 7)) < 0.8
    ok[:, 0] = True
    m = ok.sum(axis=1)
    res2, res1 = [], []
    for eps in (1e-1, 1e-2):
        z = eps * z0
        target = pisa.logsumexp(np.where(ok, z, -np.inf), axis=-1) - np.log(m)
        res2.append(np.max(np.abs(pisa.child_score(z, ok, "mean_var") - target)))
        res1.append(np.max(np.abs(pisa.child_score(z, ok, "mean") - target)))
    assert res2[1] < res2[0] * 2e-3 and res2[1] < 1e-5        # ~eps^3: 1000x smaller for 10x smaller eps
    assert 5e-3 < res1[1] / res1[0] < 2e-2                   # ~eps^2: 100x smaller
    assert np.all(pisa.child_score(np.zeros((2, 3)), np.zeros((2, 3), bool), "mean_var") == -np.inf)


def test_mean_score_without_cuts_equals_the_flat_mean_selection():
    """PISA-1 (mean of the logits) at the leaf level is linear in the keys, so when no level above the
    leaves is cut (K >= ceil(M1/2)) and every valid block is full, the hierarchy returns the flat
    mean-key selection of the block-sparse framework."""
    rng = np.random.default_rng(402)
    C, G, d, m1 = 4, 3, 6, 14
    n = C * m1
    k = rng.standard_normal((n, d))
    q = rng.standard_normal((n, G, d)) + 0.2
    K = -(-m1 // 2)
    ts = np.arange(C - 1, n, C)
    pyr = pisa.build_pyramid(k, C, 2)
    sel, _ = pisa.route(q[ts], k, pyr, ts, K, C, 2, score="mean")
    flat, gap = pisa.flat_mean_select(q[ts], pyr[0], ts, K, C)
    for r in range(len(ts)):
        if gap[r] > 1e-9:
            assert list(sel[r]) == list(flat[r]), ts[r]


# ----------------------------------------------------------------------------- gradients (R9)
def _bwd_case(seed, n=150, G=2, d=4, K=2, C=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, G, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    do = rng.standard_normal((n, G, d))
    ts = np.arange(n)
    sel, _ = pisa.route(q, k, pisa.build_pyramid(k, C), ts, K, C=C)
    return q, k, v, do, ts, sel, C


def test_attention_backward_matches_finite_differences():
    """R9: dq, dk, dv are the derivatives of L = sum(dO * O) with the selections held fixed;
    central differences of the forward oracle (fp64, step 1e-6) on every coordinate."""
    q, k, v, do, ts, sel, C = _bwd_case(0, n=40, G=2, d=3, K=1, C=8)
    dq, dk, dv = pisa.attention_backward(q, k, v, sel, ts, do, C=C)

    def loss(qq, kk, vv):
        return float(np.sum(pisa.attention(qq, kk, vv, sel, ts, C=C)[0] * do))

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if a is x else a for a in args]
            am = [xm if a is x else a for a in args]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_attention_backward_dense_equals_autograd_of_textbook_attention():
    """With every leaf selected the sparse attention is dense causal attention, so its gradients are
    torch float64 autograd of the textbook form softmax(q k^T scale + causal mask) v."""
    import torch

    n, G, d, C = 90, 3, 5, 16
    rng = np.random.default_rng(1)
    q, k, v, do = (rng.standard_normal(s) for s in ((n, G, d), (n, d), (n, d), (n, G, d)))
    ts = np.arange(n)
    m1 = -(-n // C)
    sel = np.tile(np.arange(m1), (n, 1))
    sel = np.where(sel * C <= ts[:, None], sel, -1)
    dq, dk, dv = pisa.attention_backward(q, k, v, sel, ts, do, C=C)

    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    logits = torch.einsum("tgd,sd->tgs", qt, kt) / math.sqrt(d)
    mask = torch.arange(n)[None, :] > torch.arange(n)[:, None]
    logits = logits.masked_fill(mask[:, None, :], float("-inf"))
    out = torch.einsum("tgs,sd->tgd", torch.softmax(logits, dim=-1), vt)
    out.backward(torch.tensor(do))
    for got, want in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_attention_backward_invariants(seed):
    """Closed forms of the softmax gradient: each row's dS sums to zero, so sum_r dk_r = 0; each row's
    weights sum to one, so sum_r dv_r = sum over tokens and heads of dO; rows with no key get dq = 0."""
    q, k, v, do, ts, sel, C = _bwd_case(10 + seed)
    dq, dk, dv = pisa.attention_backward(q, k, v, sel, ts, do, C=C)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=(0, 1)), rtol=1e-10, atol=1e-10)
    sel_none = sel.copy()
    sel_none[5] = -1
    dq2, _, _ = pisa.attention_backward(q, k, v, sel_none, ts, do, C=C)
    assert np.all(dq2[5] == 0.0)
    # keys no token selects get no gradient
    used = np.zeros(k.shape[0], dtype=bool)
    for r, t in enumerate(ts):
        for j in sel[r][sel[r] >= 0]:
            used[j * C:min((j + 1) * C, t + 1)] = True
    assert np.all(dk[~used] == 0.0) and np.all(dv[~used] == 0.0)
