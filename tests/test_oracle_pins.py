"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test names the page passage it pins.  No expected value here comes from
the HIP path; stored values live in tests/golden/ with their citation.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import (
    silu, swiglu_ffn, dense_ffn, router_probs, topk_canonical, renorm_weights,
    expert_lists, aux_loss, moe_route, moe_ffn,
)
from workloads import intermediate_size

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------- SiLU
def test_silu_printed_facts():
    """Chapter-4 example script, example 2: SiLU(0) = 0; minimum near
    x = -1.278 with value about -0.278."""
    g = gold("silu_facts.json")
    assert silu(np.array([0.0]))[0] == g["printed"]["silu_at_0"]
    xs = np.linspace(-3, 0, 300001)
    ys = silu(xs)
    i = int(np.argmin(ys))
    assert round(xs[i], 3) == g["printed"]["argmin_approx"]
    assert round(ys[i], 3) == g["printed"]["min_approx"]


def test_silu_closed_forms():
    """SiLU(x) = x * sigmoid(x) (chapter 4, section 4.2) at points with known
    sigmoid values, and the exact minimum x* = -1 - W(1/e), SiLU(x*) = x* + 1."""
    c = gold("silu_facts.json")["closed_form"]
    v = silu(np.array([1.0, -1.0, 2.0]))
    assert v[0] == pytest.approx(c["sigmoid_1"], rel=1e-15)
    assert v[1] == pytest.approx(-c["sigmoid_m1"], rel=1e-15)
    assert v[2] == pytest.approx(2 * c["sigmoid_2"], rel=1e-15)
    xs = np.array([c["argmin"] - 1e-4, c["argmin"], c["argmin"] + 1e-4])
    ys = silu(xs)
    assert ys[1] == pytest.approx(c["min"], abs=1e-15)
    assert ys[1] < ys[0] and ys[1] < ys[2]


def test_silu_odd_part_identity():
    """x sigmoid(x) - (-x) sigmoid(-x) = x (sigmoid(x) + sigmoid(-x)) = x:
    catches a sign error in either branch."""
    x = rnd(10000, 1, 6.0)
    np.testing.assert_allclose(silu(x) - silu(-x), x, rtol=1e-14, atol=1e-15)


def test_silu_extremes_finite():
    v = silu(np.array([-800.0, 800.0, -40.0]))
    assert np.all(np.isfinite(v))
    assert v[1] == 800.0 and v[0] == 0.0 and -1e-15 < v[2] < 0


# ------------------------------------------------------------ dense FFN
@pytest.mark.parametrize("case", gold("swiglu_hand.json")["cases"], ids=lambda c: c["name"])
def test_swiglu_hand_cases(case):
    """Lesson 13 sections 0/1.2: y = W_down(SiLU(W_gate x) * W_up x), weights
    [out, in].  Hand-derived values (gate/up swap and transposes fail these)."""
    y = swiglu_ffn(np.array(case["x"]), np.array(case["Wg"]), np.array(case["Wu"]), np.array(case["Wd"]))
    np.testing.assert_allclose(y, np.array(case["y"]), rtol=1e-14)


def test_dense_zero_up_projection():
    x = rnd((5, 8), 2)
    y = swiglu_ffn(x, rnd((12, 8), 3), np.zeros((12, 8)), rnd((8, 12), 4))
    assert np.all(y == 0)


def test_dense_rows_are_independent():
    """The FFN transforms each token on its own (lesson 13, section 1.1)."""
    x, Wg, Wu, Wd = rnd((9, 8), 5), rnd((6, 8), 6), rnd((6, 8), 7), rnd((8, 6), 8)
    full = dense_ffn(x, Wg, Wu, Wd)
    rows = [7, 0, 3]
    np.testing.assert_allclose(dense_ffn(x, Wg, Wu, Wd, rows=rows), full[rows], rtol=1e-14)


def test_intermediate_size_formula():
    """Config default ceil(H * pi / 64) * 64 (lesson 13 section 3 step 1):
    chapter 4 section 4.1 prints 2432 for H = 768."""
    assert intermediate_size(768) == 2432
    assert intermediate_size(2048) == 6464


# ------------------------------------------------------ router / top-k
def test_softmax_sums_to_one_and_shift_invariant():
    """p = softmax(W_router x) (lesson 13 section 1.5): a distribution, and
    unchanged by a constant added to every logit."""
    x = rnd((50, 16), 9)
    Wr = rnd((8, 16), 10, 0.3)
    p = router_probs(x, Wr)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-15)
    x1 = np.concatenate([x, np.ones((50, 1))], axis=1)
    Wr1 = np.concatenate([Wr, np.full((8, 1), 7.5)], axis=1)
    np.testing.assert_allclose(router_probs(x1, Wr1), p, rtol=1e-13)


def test_softmax_zero_router_uniform():
    for E in (1, 2, 4, 8, 64):
        p = router_probs(rnd((7, 16), 11), np.zeros((E, 16)))
        assert np.all(p == 1.0 / E)


def test_softmax_recovers_worked_probabilities():
    """Logits log(p) reproduce the worked p of lesson 13 section 1.5."""
    g = gold("routing_worked_example.json")
    p = np.array(g["p"])
    got = router_probs(np.ones((1, 1)), np.log(p)[:, None])
    np.testing.assert_allclose(got[0], p, rtol=1e-14)


@pytest.mark.parametrize("case", gold("routing_worked_example.json")["cases"], ids=lambda c: f"k{c['k']}")
def test_topk_and_alpha_worked_example(case):
    """Lesson 13 section 1.5 worked routing (top-1 -> {2}; top-2 -> {2,1}
    with alpha = 0.8/0.9, 0.1/0.9); top-3 under the lower-id tie reading."""
    p = np.array([gold("routing_worked_example.json")["p"]])
    idx = topk_canonical(p, case["k"])
    assert idx[0].tolist() == case["topk_idx"]
    alpha = renorm_weights(p, idx)
    np.testing.assert_allclose(alpha[0], case["alpha"], rtol=1e-14)


def test_topk_brute_force_subsets():
    """TopK(p, k) is the k-subset of largest total probability (lesson 13
    section 0), listed in descending probability; checked against every subset."""
    rng = np.random.default_rng(12)
    for E in (2, 3, 5, 8):
        for _ in range(40):
            p = rng.dirichlet(np.ones(E))[None, :]
            for k in range(1, E + 1):
                idx = topk_canonical(p, k)[0]
                best = max(itertools.combinations(range(E), k), key=lambda s: p[0, list(s)].sum())
                assert sorted(idx.tolist()) == sorted(best)
                assert np.all(np.diff(p[0, idx]) <= 0)


def test_topk_tie_goes_to_lower_id():
    p = np.array([[0.25, 0.25, 0.25, 0.25], [0.1, 0.4, 0.1, 0.4]])
    assert topk_canonical(p, 2).tolist() == [[0, 1], [1, 3]]


@pytest.mark.parametrize("case", gold("routing_worked_example.json")["raw_cases"], ids=lambda c: f"k{c['k']}")
def test_alpha_raw_without_renormalisation(case):
    """norm_topk_prob False (lesson 13 section 3 step 5; chapter 4 section 4.3
    step 2): alpha is the selected probabilities, the printed 0.80 and 0.10."""
    p = np.array([gold("routing_worked_example.json")["p"]])
    idx = topk_canonical(p, case["k"])
    assert idx[0].tolist() == case["topk_idx"]
    alpha = renorm_weights(p, idx, normalize=False)
    np.testing.assert_array_equal(alpha[0], case["alpha"])
    r = moe_route(np.ones((1, 1)), np.log(p[0])[:, None], case["k"], 0.0, norm_topk_prob=False)
    np.testing.assert_allclose(r["alpha"][0], case["alpha"], rtol=1e-14)


def test_alpha_raw_sums_below_one_unless_all_experts():
    """Without renormalisation sum_j alpha = sum of the selected p: below 1 for
    k < E, 1 (up to rounding) for k = E, and the top-k set is unchanged."""
    p = router_probs(rnd((100, 32), 31), rnd((6, 32), 32, 0.5))
    for k in (1, 3, 6):
        idx = topk_canonical(p, k)
        a = renorm_weights(p, idx, normalize=False)
        if k < 6:
            assert np.all(a.sum(1) < 1.0)
        else:
            np.testing.assert_allclose(a.sum(1), 1.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(a / a.sum(1, keepdims=True), renorm_weights(p, idx), rtol=1e-12)


def test_alpha_sums_to_one_and_top1_is_one():
    """norm_topk_prob renormalisation (lesson 13 section 3 step 5; chapter-4
    example 6 checks the sum against 1 with atol 1e-5); k = 1 gives 1 exactly."""
    p = router_probs(rnd((200, 32), 13), rnd((8, 32), 14, 0.5))
    for k in (1, 2, 3, 8):
        a = renorm_weights(p, topk_canonical(p, k))
        np.testing.assert_allclose(a.sum(1), 1.0, rtol=0, atol=1e-12)
        if k == 1:
            assert np.all(a == 1.0)


# ------------------------------------------------------- residual stream
def test_residual_with_zero_down_projection_is_the_residual():
    """hidden_states + mlp(...) (lesson 13 section 1.3): W_down = 0 makes the
    FFN output 0, so y is the residual exactly (dense and MoE)."""
    x, R = rnd((9, 16), 41), rnd((9, 16), 42)
    Wg, Wu = rnd((24, 16), 43, 0.3), rnd((24, 16), 44, 0.3)
    y = dense_ffn(x, Wg, Wu, np.zeros((16, 24)), residual=R)
    np.testing.assert_array_equal(y, R)
    Wr = rnd((3, 16), 45, 0.5)
    out = moe_ffn(x, Wr, rnd((3, 24, 16), 46, 0.3), rnd((3, 24, 16), 47, 0.3),
                  np.zeros((3, 16, 24)), 2, 0.01, residual=R)
    np.testing.assert_array_equal(out["y"], R)


def test_residual_rows_subset_and_single_expert():
    """The residual is added on each token's own row: a row subset of the full
    result, and E = k = 1 equals the dense FFN with the same residual."""
    x, R = rnd((12, 16), 51), rnd((12, 16), 52)
    Wg, Wu, Wd = rnd((1, 24, 16), 53, 0.3), rnd((1, 24, 16), 54, 0.3), rnd((1, 16, 24), 55, 0.3)
    Wr = rnd((1, 16), 56)
    full = moe_ffn(x, Wr, Wg, Wu, Wd, 1, 0.0, residual=R)["y"]
    rows = [7, 2, 11]
    sub_y = moe_ffn(x, Wr, Wg, Wu, Wd, 1, 0.0, rows=rows, residual=R)["y"]
    np.testing.assert_array_equal(sub_y, full[rows])
    dense = dense_ffn(x, Wg[0], Wu[0], Wd[0], residual=R)
    np.testing.assert_allclose(full, dense, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(dense_ffn(x, Wg[0], Wu[0], Wd[0], rows=rows, residual=R),
                                  dense[rows])


# ---------------------------------------------------- per-expert lists
def test_expert_lists_invariants():
    """Per-expert token lists (lesson 13 section 3 step 5): sum of counts is
    N*k; each list strictly ascending; t in L_e iff e in S_t."""
    N, E = 300, 8
    p = router_probs(rnd((N, 16), 15), rnd((E, 16), 16, 0.6))
    for k in (1, 2, 5):
        idx = topk_canonical(p, k)
        counts, offsets, ids = expert_lists(idx, E)
        assert counts.sum() == N * k and offsets[-1] == N * k
        assert np.all(np.diff(offsets) == counts)
        for e in range(E):
            L = ids[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(L) > 0)
            chose = np.nonzero((idx == e).any(1))[0]
            assert L.tolist() == chose.tolist()


# -------------------------------------------------------------- MoE y
def _experts(E, H, I, seed):
    return rnd((E, I, H), seed, 0.3), rnd((E, I, H), seed + 1, 0.3), rnd((E, H, I), seed + 2, 0.3)


def test_moe_k_equals_E_is_dense_weighted_sum():
    """With k = E every expert is selected and alpha = p (their sum is 1), so
    y = sum_e p_e Expert_e(x) (lesson 13 section 0; study notes section 9)."""
    N, H, I, E = 17, 12, 10, 5
    x, Wr = rnd((N, H), 20), rnd((E, H), 21, 0.5)
    Wg, Wu, Wd = _experts(E, H, I, 22)
    res = moe_ffn(x, Wr, Wg, Wu, Wd, k=E, coef=0.0)
    p = router_probs(x, Wr)
    brute = sum(p[:, e:e + 1] * swiglu_ffn(x, Wg[e], Wu[e], Wd[e]) for e in range(E))
    np.testing.assert_allclose(res["y"], brute, rtol=1e-12, atol=1e-14)


def test_moe_single_expert_is_dense():
    N, H, I = 11, 8, 6
    x = rnd((N, H), 23)
    Wg, Wu, Wd = _experts(1, H, I, 24)
    res = moe_ffn(x, rnd((1, H), 25), Wg, Wu, Wd, k=1, coef=0.01)
    np.testing.assert_allclose(res["y"], swiglu_ffn(x, Wg[0], Wu[0], Wd[0]), rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_moe_identical_experts_is_dense(k):
    """Identical experts: y = (sum_j alpha_j) FFN(x) = FFN(x) for any routing."""
    N, H, I, E = 13, 8, 6, 4
    x = rnd((N, H), 26)
    Wg, Wu, Wd = _experts(1, H, I, 27)
    rep = lambda W: np.repeat(W, E, axis=0)
    res = moe_ffn(x, rnd((E, H), 28), rep(Wg), rep(Wu), rep(Wd), k=k, coef=0.01)
    np.testing.assert_allclose(res["y"], swiglu_ffn(x, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_moe_dispatch_matches_masked_brute_force(k):
    """Gather / run / scale / index_add dispatch (lesson 13 section 3 step 5)
    equals evaluating every expert on every token and keeping the selected
    ones with their alpha (no gathering)."""
    N, H, I, E = 40, 10, 7, 6
    x, Wr = rnd((N, H), 29), rnd((E, H), 30, 0.8)
    Wg, Wu, Wd = _experts(E, H, I, 31)
    res = moe_ffn(x, Wr, Wg, Wu, Wd, k=k, coef=0.01)
    p = router_probs(x, Wr)
    idx = topk_canonical(p, k)
    alpha = renorm_weights(p, idx)
    brute = np.zeros((N, H))
    for t in range(N):
        for e in range(E):
            if e in idx[t]:
                a = alpha[t, list(idx[t]).index(e)]
                brute[t] += a * swiglu_ffn(x[t:t + 1], Wg[e], Wu[e], Wd[e])[0]
    np.testing.assert_allclose(res["y"], brute, rtol=1e-12, atol=1e-14)


def test_moe_token_permutation_equivariant():
    """Tokens never mix (lesson 13 section 1.1): permuting tokens permutes y,
    topk_idx and alpha; aux only changes by summation order."""
    N, H, I, E, k = 50, 8, 6, 4, 2
    x, Wr = rnd((N, H), 32), rnd((E, H), 33, 0.8)
    Wg, Wu, Wd = _experts(E, H, I, 34)
    a = moe_ffn(x, Wr, Wg, Wu, Wd, k=k, coef=0.01)
    perm = np.random.default_rng(35).permutation(N)
    b = moe_ffn(x[perm], Wr, Wg, Wu, Wd, k=k, coef=0.01)
    np.testing.assert_allclose(b["y"], a["y"][perm], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(b["topk_idx"], a["topk_idx"][perm])
    np.testing.assert_allclose(b["alpha"], a["alpha"][perm], rtol=1e-15)
    assert b["aux"] == pytest.approx(a["aux"], rel=1e-13)


def test_moe_rows_subset():
    N, H, I, E, k = 30, 8, 6, 4, 2
    x, Wr = rnd((N, H), 36), rnd((E, H), 37, 0.8)
    Wg, Wu, Wd = _experts(E, H, I, 38)
    full = moe_ffn(x, Wr, Wg, Wu, Wd, k=k, coef=0.01)
    rows = [29, 3, 4, 17]
    sub = moe_ffn(x, Wr, Wg, Wu, Wd, k=k, coef=0.01, rows=rows)
    np.testing.assert_allclose(sub["y"], full["y"][rows], rtol=1e-13, atol=1e-16)


# ---------------------------------------------------------------- aux
@pytest.mark.parametrize("case", gold("aux_extremes.json")["cases"], ids=lambda c: c["name"])
def test_aux_worked_extremes(case):
    """Chapter 4 section 4.4 table: balanced E*sum(fP) = 1.0; collapsed 2.8.
    Realised with N = 4 tokens, top-1, every token's p equal to P."""
    E, coef = 4, 0.5
    P = np.array(case["P"])
    f = np.array(case["f"])
    N = 4
    idx = np.repeat(np.arange(E), (f * N).astype(int))[:, None]
    p = np.tile(P, (N, 1))
    assert aux_loss(p, idx, E, coef) == pytest.approx(case["aux_over_coef"] * coef, rel=1e-15)


def test_aux_closed_form():
    """aux = coef * E * sum_e c_e * s_e / N^2 with s_e = sum_t p_{t,e}
    (lesson 13 section 1.6 equation with load_e = c_e / N)."""
    N, E = 123, 8
    p = router_probs(rnd((N, 16), 40), rnd((E, 16), 41, 0.7))
    for k in (1, 2, 3):
        idx = topk_canonical(p, k)
        counts, _, _ = expert_lists(idx, E)
        closed = 0.01 * E * float((counts * p.sum(0)).sum()) / N**2
        assert aux_loss(p, idx, E, 0.01) == pytest.approx(closed, rel=1e-13)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_aux_uniform_router_is_k_coef(K):
    """W_router = 0: every p = 1/E, ties pick experts 0..K-1, and the module's
    [K, E] load gives aux = K * coef exactly (coef for the default K = 1)."""
    E, coef = 8, 0.01
    r = moe_route(rnd((64, 16), 42), np.zeros((E, 16)), K, coef)
    assert r["aux"] == K * coef


@pytest.mark.parametrize("K", [1, 2, 3])
def test_aux_cyclic_balanced_routing(K):
    """Perfectly balanced loads (c_e = N K / E) with mean probabilities 1/E
    give aux = K * coef up to rounding."""
    E, N, coef = 4, 64, 0.01
    q = np.array([0.4, 0.3, 0.2, 0.1])
    p = np.stack([np.roll(q, t) for t in range(N)])
    idx = np.stack([(np.arange(K) + t) % E for t in range(N)])
    assert aux_loss(p, idx, E, coef) == pytest.approx(K * coef, rel=1e-14)


def test_aux_nonnegative_and_disabled():
    """Example 7 asserts aux >= 0; coef = 0 is the disabled branch (zero)."""
    p = router_probs(rnd((77, 16), 43), rnd((6, 16), 44))
    idx = topk_canonical(p, 2)
    assert aux_loss(p, idx, 6, 0.01) >= 0
    assert aux_loss(p, idx, 6, 0.0) == 0.0
