"""Pins of the oracle's backward pass to facts other than its own formulas.

The backward is the gradient of the forward (the top-k choice and the expert
counts carry none; the softmax probabilities do, through the selected weights
and through aux -- chapter 4, section 4.4 and the study notes' section 7 on
how the router is trained).  Pinned here by:
  * central finite differences of the oracle's FORWARD, element by element,
    on shapes where every dimension differs (a transposed or dropped term
    fails), in both weight modes and with aux on and off;
  * SiLU' at the printed facts of example 2 (SiLU' = 1/2 at 0, SiLU' = 0 at
    the minimum) and its limits;
  * special cases: one expert with k = 1 is the dense FFN (and the router gets
    nothing); identical experts with k = E make y independent of the router;
    linearity in the upstream gradient.
"""
import json
import os

import numpy as np
import pytest

from oracle import (
    silu, silu_grad, swiglu_ffn, swiglu_ffn_bwd, moe_ffn, moe_ffn_bwd, moe_ffn_bwd_sampled,
    router_probs, topk_canonical,
)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def fd_grad(f, params, name, h=1e-6):
    """Central difference of scalar f(params) w.r.t. every element of
    params[name]."""
    base = params[name]
    g = np.zeros_like(base)
    for i in np.ndindex(base.shape):
        old = base[i]
        base[i] = old + h
        fp = f(params)
        base[i] = old - h
        fm = f(params)
        base[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


# ------------------------------------------------------------------ SiLU'
def test_silu_grad_printed_facts():
    """Example 2 of the chapter-4 example script: SiLU passes the origin with
    slope 1/2 and has its minimum near -1.278, where the slope is zero."""
    with open(os.path.join(GOLD, "silu_facts.json")) as f:
        c = json.load(f)["closed_form"]
    assert silu_grad(np.array([0.0]))[0] == 0.5
    assert abs(silu_grad(np.array([c["argmin"]]))[0]) < 1e-15
    # sign change around the minimum
    assert silu_grad(np.array([c["argmin"] - 1e-3]))[0] < 0 < silu_grad(np.array([c["argmin"] + 1e-3]))[0]


def test_silu_grad_limits_and_fd():
    z = np.linspace(-30, 30, 601)
    h = 1e-6
    fd = (silu(z + h) - silu(z - h)) / (2 * h)
    np.testing.assert_allclose(silu_grad(z), fd, rtol=1e-7, atol=1e-8)
    assert silu_grad(np.array([60.0]))[0] == pytest.approx(1.0, abs=1e-20)
    assert abs(silu_grad(np.array([-60.0]))[0]) < 1e-20
    assert np.isfinite(silu_grad(np.array([-800.0, 800.0]))).all()


# ------------------------------------------------------- dense SwiGLU bwd
def test_swiglu_bwd_finite_differences():
    T, H, I = 3, 5, 4
    P = {"x": rnd((T, H), 1), "Wg": rnd((I, H), 2, 0.5), "Wu": rnd((I, H), 3, 0.5),
         "Wd": rnd((H, I), 4, 0.5)}
    dy = rnd((T, H), 5)

    def L(q):
        return float((dy * swiglu_ffn(q["x"], q["Wg"], q["Wu"], q["Wd"])).sum())

    dx, dWg, dWu, dWd = swiglu_ffn_bwd(P["x"], P["Wg"], P["Wu"], P["Wd"], dy)
    for name, got in (("x", dx), ("Wg", dWg), ("Wu", dWu), ("Wd", dWd)):
        assert got.shape == P[name].shape
        np.testing.assert_allclose(got, fd_grad(L, P, name), rtol=1e-6, atol=1e-8, err_msg=name)


def test_swiglu_bwd_zero_and_linearity():
    T, H, I = 4, 3, 6
    x, Wg, Wu, Wd = rnd((T, H), 11), rnd((I, H), 12), rnd((I, H), 13), rnd((H, I), 14)
    for a in swiglu_ffn_bwd(x, Wg, Wu, Wd, np.zeros((T, H))):
        assert not a.any()
    d1, d2 = rnd((T, H), 15), rnd((T, H), 16)
    g1 = swiglu_ffn_bwd(x, Wg, Wu, Wd, d1)
    g2 = swiglu_ffn_bwd(x, Wg, Wu, Wd, d2)
    g3 = swiglu_ffn_bwd(x, Wg, Wu, Wd, d1 - 3.0 * d2)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, a - 3.0 * b, rtol=1e-12, atol=1e-12)


def test_swiglu_bwd_rows_independent():
    """Each token's dx depends on its own row only; weight grads add over
    tokens (the FFN acts on each position on its own, section 4.2)."""
    T, H, I = 5, 4, 3
    x, Wg, Wu, Wd, dy = rnd((T, H), 21), rnd((I, H), 22), rnd((I, H), 23), rnd((H, I), 24), rnd((T, H), 25)
    full = swiglu_ffn_bwd(x, Wg, Wu, Wd, dy)
    parts = [swiglu_ffn_bwd(x[t:t + 1], Wg, Wu, Wd, dy[t:t + 1]) for t in range(T)]
    np.testing.assert_allclose(full[0], np.concatenate([p[0] for p in parts]), rtol=1e-13, atol=1e-14)
    for j in (1, 2, 3):
        np.testing.assert_allclose(full[j], sum(p[j] for p in parts), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- MoE bwd
def _moe_params(N, H, I, E, seed):
    return {"x": rnd((N, H), seed), "Wr": rnd((E, H), seed + 1, 0.7),
            "Wg": rnd((E, I, H), seed + 2, 0.5), "Wu": rnd((E, I, H), seed + 3, 0.5),
            "Wd": rnd((E, H, I), seed + 4, 0.5)}


def _margin(x, Wr, k):
    """Smallest gap between the k-th and (k+1)-th probability over tokens."""
    p = np.sort(router_probs(x, Wr), axis=1)[:, ::-1]
    if k >= p.shape[1]:
        return np.inf
    return float((p[:, k - 1] - p[:, k]).min())


@pytest.mark.parametrize("k,coef,norm", [(1, 0.0, True), (2, 0.0, True), (2, 0.1, True),
                                         (2, 0.1, False), (3, 0.05, False), (1, 0.3, True)])
def test_moe_bwd_finite_differences(k, coef, norm):
    """Every gradient of moe_ffn_bwd against central differences of
    L = sum(dy * y) + daux * aux_loss, computed with the forward only.  The
    seed is checked to keep the top-k choice away from ties, where the
    forward is not differentiable."""
    N, H, I, E = 7, 5, 3, 4
    seed = 100 + 10 * k
    P = _moe_params(N, H, I, E, seed)
    while _margin(P["x"], P["Wr"], k) <= 1e-3:
        seed += 1
        P = _moe_params(N, H, I, E, seed)
    dy = rnd((N, H), 7)
    daux = 1.7

    def L(q):
        r = moe_ffn(q["x"], q["Wr"], q["Wg"], q["Wu"], q["Wd"], k, coef, norm_topk_prob=norm)
        return float((dy * r["y"]).sum()) + daux * r["aux"]

    idx0 = topk_canonical(router_probs(P["x"], P["Wr"]), k)
    g = moe_ffn_bwd(P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], k, coef, dy, daux, norm)
    assert np.array_equal(g["route"]["topk_idx"], idx0)
    for name, key in (("x", "dx"), ("Wr", "dWr"), ("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd")):
        assert g[key].shape == P[name].shape
        np.testing.assert_allclose(g[key], fd_grad(L, P, name), rtol=1e-6, atol=1e-8, err_msg=name)


def test_moe_bwd_one_expert_is_dense():
    """E = k = 1: every token goes to the single expert with weight 1, so the
    MoE backward is the dense one and the router, whose softmax is constant,
    gets zero gradient even with aux on."""
    N, H, I = 6, 4, 5
    P = _moe_params(N, H, I, 1, 300)
    dy = rnd((N, H), 9)
    g = moe_ffn_bwd(P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], 1, 0.1, dy, 1.0, True)
    d = swiglu_ffn_bwd(P["x"], P["Wg"][0], P["Wu"][0], P["Wd"][0], dy)
    np.testing.assert_allclose(g["dx"], d[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dWg"][0], d[1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dWu"][0], d[2], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dWd"][0], d[3], rtol=1e-13, atol=1e-14)
    assert np.abs(g["dWr"]).max() < 1e-15


@pytest.mark.parametrize("norm", [True, False])
def test_moe_bwd_identical_experts_all_selected(norm):
    """k = E with every expert the same: y = (sum of the weights) * FFN(x),
    and that sum is 1 (up to the 1e-20 guard) in both weight modes, so y
    does not depend on the router.  Without aux the router gets no gradient;
    dx and the summed expert gradients are the dense ones."""
    N, H, I, E = 5, 4, 3, 3
    P = _moe_params(N, H, I, E, 400)
    for w in ("Wg", "Wu", "Wd"):
        P[w][:] = P[w][0]
    dy = rnd((N, H), 10)
    g = moe_ffn_bwd(P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], E, 0.0, dy, 0.0, norm)
    d = swiglu_ffn_bwd(P["x"], P["Wg"][0], P["Wu"][0], P["Wd"][0], dy)
    assert np.abs(g["dWr"]).max() < 1e-13
    np.testing.assert_allclose(g["dx"], d[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWg"].sum(0), d[1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWu"].sum(0), d[2], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWd"].sum(0), d[3], rtol=1e-11, atol=1e-12)


def test_moe_bwd_unselected_expert_gets_nothing():
    """An expert no token selects gets zero weight gradients (study notes
    section 7: unselected experts are not updated by this batch)."""
    N, H, I, E = 6, 4, 3, 4
    P = _moe_params(N, H, I, E, 500)
    P["Wr"][3] = -50.0 * np.sign(P["x"].mean(0))     # expert 3 never wins
    P["x"] = np.abs(P["x"]) * np.sign(P["x"].mean(0))
    dy = rnd((N, H), 11)
    g = moe_ffn_bwd(P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], 2, 0.1, dy, 1.0, True)
    assert not (g["route"]["topk_idx"] == 3).any()
    for key in ("dWg", "dWu", "dWd"):
        assert not g[key][3].any()
        assert g[key][:3].any()


def test_moe_bwd_linearity_and_zero():
    N, H, I, E, k = 6, 4, 3, 4, 2
    P = _moe_params(N, H, I, E, 600)
    args = (P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], k, 0.1)
    z = moe_ffn_bwd(*args, np.zeros((N, H)), 0.0, True)
    for key in ("dx", "dWr", "dWg", "dWu", "dWd"):
        assert not z[key].any()
    d1, d2 = rnd((N, H), 12), rnd((N, H), 13)
    a = moe_ffn_bwd(*args, d1, 1.0, True)
    b = moe_ffn_bwd(*args, d2, 2.0, True)
    c = moe_ffn_bwd(*args, d1 + 0.5 * d2, 2.0, True)
    for key in ("dx", "dWr", "dWg", "dWu", "dWd"):
        np.testing.assert_allclose(c[key], a[key] + 0.5 * b[key], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("k,coef,norm", [(1, 0.01, True), (2, 0.05, False), (3, 0.02, True)])
def test_moe_bwd_sampled_matches_full(k, coef, norm):
    """The sampled entry point (dx row by row, weight gradients of a subset of
    intermediate units) reproduces the corresponding parts of the full backward."""
    N, H, I, E = 40, 6, 7, 5
    P = _moe_params(N, H, I, E, 700 + k)
    dy = rnd((N, H), 17)
    args = (P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], k, coef, dy, 1.3, norm)
    full = moe_ffn_bwd(*args)
    rows = np.array([0, 3, 17, 39])
    units = np.array([1, 4, 6])
    s = moe_ffn_bwd_sampled(*args, rows=rows, units=units)
    np.testing.assert_allclose(s["dx_rows"], full["dx"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dWg_u"], full["dWg"][:, units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dWu_u"], full["dWu"][:, units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dWd_u"], full["dWd"][:, :, units], rtol=1e-12, atol=1e-13)


def test_moe_bwd_sampled_all_rows_gives_dwr():
    N, H, I, E = 30, 5, 6, 4
    P = _moe_params(N, H, I, E, 800)
    dy = rnd((N, H), 18)
    args = (P["x"], P["Wr"], P["Wg"], P["Wu"], P["Wd"], 2, 0.03, dy, 0.7, True)
    full = moe_ffn_bwd(*args)
    s = moe_ffn_bwd_sampled(*args, units=np.array([0, 5]))
    np.testing.assert_allclose(s["dWr"], full["dWr"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dx_rows"], full["dx"], rtol=1e-12, atol=1e-13)
    assert moe_ffn_bwd_sampled(*args, rows=[1, 2])["dWr"] is None
