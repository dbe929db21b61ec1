"""Pins of the oracle's router z-loss and expert capacity.

The pages name both without defining them (the study notes' section 10
table; lesson 13 section 4 lists capacity / token dropping as not required),
so the definitions are readings of the standard forms: z-loss = z_coef *
mean_t logsumexp(r_t)^2; capacity C = ceil(factor * N * k / E), each expert
keeps its first C tokens in ascending token order.  What is pinned here is
the oracle against those definitions, by closed forms, a library routine,
brute force written differently, and finite differences of the forward.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import (expert_capacity, kept_entries, logsumexp_rows, moe_ffn, moe_ffn_bwd,
                    moe_route, router_probs, router_z_loss, swiglu_ffn)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ z-loss
def test_logsumexp_matches_library_and_is_overflow_safe():
    r = rnd((50, 7), 1, 5.0)
    np.testing.assert_allclose(logsumexp_rows(r), logsumexp(r, axis=1), rtol=1e-14)
    big = np.full((3, 4), 1000.0)
    np.testing.assert_allclose(logsumexp_rows(big), 1000.0 + np.log(4.0), rtol=1e-15)
    np.testing.assert_allclose(logsumexp_rows(r + 3.5), logsumexp_rows(r) + 3.5, rtol=1e-13)


def test_z_loss_closed_forms():
    x = rnd((20, 6), 2)
    E = 5
    # W_r = 0: every logit 0, logsumexp = log E
    assert router_z_loss(x, np.zeros((E, 6)), 0.25) == pytest.approx(0.25 * np.log(E) ** 2,
                                                                     rel=1e-14)
    # one expert: logsumexp is the logit itself
    Wr = rnd((1, 6), 3)
    r = x @ Wr.T
    assert router_z_loss(x, Wr, 0.1) == pytest.approx(0.1 * np.mean(r[:, 0] ** 2), rel=1e-13)
    assert router_z_loss(x, rnd((E, 6), 4), 0.0) == 0.0
    r = moe_route(x, rnd((E, 6), 4), 2, 0.01, z_coef=0.3)
    assert r["z_loss"] == pytest.approx(0.3 * np.mean(logsumexp(x @ rnd((E, 6), 4).T, axis=1) ** 2))


# ---------------------------------------------------------------- capacity
def test_capacity_values():
    assert expert_capacity(10, 2, 4, 1.0) == 5
    assert expert_capacity(10, 2, 4, 1.25) == 7      # ceil(6.25)
    assert expert_capacity(3, 1, 8, 0.5) == 1         # ceil(0.1875)
    assert expert_capacity(100, 1, 4, 0.0) is None


def test_kept_entries_brute_force():
    """Stream the tokens in ascending order with one counter per expert: a
    pair is kept while its expert has taken fewer than C tokens."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        N, E, k = int(rng.integers(1, 40)), int(rng.integers(1, 7)), 0
        k = int(rng.integers(1, E + 1))
        idx = np.array([rng.permutation(E)[:k] for _ in range(N)])
        C = int(rng.integers(0, N + 2))
        taken = np.zeros(E, dtype=int)
        want = np.zeros((N, k), dtype=bool)
        for t in range(N):
            for j in range(k):
                e = idx[t, j]
                want[t, j] = taken[e] < C
                taken[e] += 1
        np.testing.assert_array_equal(kept_entries(idx, E, C), want)
    assert kept_entries(idx, E, None).all()


def _params(N, H, I, E, seed):
    return (rnd((N, H), seed), rnd((E, H), seed + 1, 0.7), rnd((E, I, H), seed + 2, 0.5),
            rnd((E, I, H), seed + 3, 0.5), rnd((E, H, I), seed + 4, 0.5))


def test_capacity_forward_brute_force():
    """y_t = residual_t + sum over the kept slots of alpha * Expert(x_t),
    token by token; aux uses the choices before dropping."""
    N, H, I, E, k = 40, 5, 6, 4, 2
    x, Wr, Wg, Wu, Wd = _params(N, H, I, E, 10)
    res = rnd((N, H), 15)
    for cf in (0.5, 0.8, 1.0):
        out = moe_ffn(x, Wr, Wg, Wu, Wd, k, 0.01, residual=res, capacity_factor=cf)
        C = expert_capacity(N, k, E, cf)
        keep = kept_entries(out["topk_idx"], E, C)
        y = res.copy()
        for t in range(N):
            for j in range(k):
                if keep[t, j]:
                    e = out["topk_idx"][t, j]
                    y[t] += out["alpha"][t, j] * swiglu_ffn(x[t:t + 1], Wg[e], Wu[e], Wd[e])[0]
        np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-13)
        assert out["aux"] == pytest.approx(moe_ffn(x, Wr, Wg, Wu, Wd, k, 0.01)["aux"], rel=1e-15)
        np.testing.assert_array_equal(out["kept_counts"], np.minimum(out["counts"], C))
        assert out["kept_offsets"][-1] == keep.sum()
    # a capacity no expert reaches changes nothing
    free = moe_ffn(x, Wr, Wg, Wu, Wd, k, 0.01, residual=res, capacity_factor=float(E))
    base = moe_ffn(x, Wr, Wg, Wu, Wd, k, 0.01, residual=res)
    np.testing.assert_array_equal(free["y"], base["y"])
    np.testing.assert_array_equal(free["kept_sorted_token_ids"], base["sorted_token_ids"])


def _margin_seed(N, H, I, E, k, seed):
    while True:
        P = _params(N, H, I, E, seed)
        p = np.sort(router_probs(P[0], P[1]), axis=1)[:, ::-1]
        if k >= E or (p[:, k - 1] - p[:, k]).min() > 1e-3:
            return P
        seed += 1


def fd(f, arr, h=1e-6):
    g = np.zeros_like(arr)
    for i in np.ndindex(arr.shape):
        old = arr[i]
        arr[i] = old + h
        a = f()
        arr[i] = old - h
        b = f()
        arr[i] = old
        g[i] = (a - b) / (2 * h)
    return g


@pytest.mark.parametrize("k,cf,zc,norm", [(2, 0.0, 0.05, True), (2, 0.6, 0.0, True),
                                          (1, 0.5, 0.1, True), (2, 0.7, 0.02, False)])
def test_bwd_with_z_loss_and_capacity_finite_differences(k, cf, zc, norm):
    """Gradients of L = sum(dy * y) + daux * aux + dz * z_loss under a
    capacity, against central differences of the forward."""
    N, H, I, E = 12, 4, 3, 4
    x, Wr, Wg, Wu, Wd = _margin_seed(N, H, I, E, k, 40 + k)
    dy = rnd((N, H), 41)
    daux, dz = 1.3, 0.7

    def L():
        r = moe_ffn(x, Wr, Wg, Wu, Wd, k, 0.02, norm_topk_prob=norm, z_coef=zc, capacity_factor=cf)
        return float((dy * r["y"]).sum()) + daux * r["aux"] + dz * r["z_loss"]

    g = moe_ffn_bwd(x, Wr, Wg, Wu, Wd, k, 0.02, dy, daux, norm, z_coef=zc, dz=dz,
                    capacity_factor=cf)
    if cf:
        assert not g["route"]["keep"].all()  # the case drops something
    for name, arr in (("dx", x), ("dWr", Wr), ("dWg", Wg), ("dWu", Wu), ("dWd", Wd)):
        np.testing.assert_allclose(g[name], fd(L, arr), rtol=1e-6, atol=1e-8, err_msg=name)
