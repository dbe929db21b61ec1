"""Helpers for the GPU parity tests: move generator output to the device, call
the library, and measure the deviations from the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

TOL_Y = {"fp32": 1e-5, "bf16": 2e-2}   # max per-token relative L2 error of y
TOL_ALPHA = 1e-5                      # relative, per entry
TOL_AUX = 1e-5                        # relative


def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def announce(msg: str) -> None:
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inputs: dict, dev):
    import torch

    dt = inputs["dtype"]

    def t(a, stored=True):
        if stored and dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    out = {n: t(inputs[n]) for n in ("x", "Wg", "Wu", "Wd", "residual") if n in inputs}
    if "Wr" in inputs:
        out["Wr"] = t(inputs["Wr"], stored=False)
    return out


def y_to_f64(y) -> np.ndarray:
    import torch

    return y.detach().to(torch.float64).cpu().numpy()


def rel_l2_per_token(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if got.size else 0.0


def rel_l2_global(got: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (d if d else 1.0))


def run_moe(tm, dev_in, w, N=None, y=None):
    return tm.moe_ffn_fwd(dev_in["x"], dev_in["Wr"], dev_in["Wg"], dev_in["Wu"], dev_in["Wd"],
                          w.k, w.coef, residual=dev_in.get("residual"),
                          norm_topk_prob=w.norm_topk_prob, y=y)


def run_dense(tm, dev_in, y=None):
    return tm.ffn_swiglu_fwd(dev_in["x"], dev_in["Wg"], dev_in["Wu"], dev_in["Wd"],
                             residual=dev_in.get("residual"), y=y)


def check_routing(out, ref, k, E, exact_order=True):
    """topk_idx, per-expert lists bit-exact; alpha and aux to their tolerances."""
    idx = out.topk_idx.cpu().numpy()
    alpha = out.alpha.cpu().numpy().astype(np.float64)
    if exact_order:
        np.testing.assert_array_equal(idx, ref["topk_idx"])
        np.testing.assert_allclose(alpha, ref["alpha"], rtol=TOL_ALPHA, atol=0)
    else:
        # k == E: the selected set is every expert; compare per expert id
        oi = np.argsort(idx, axis=1)
        ri = np.argsort(ref["topk_idx"], axis=1)
        np.testing.assert_array_equal(np.take_along_axis(idx, oi, 1),
                                      np.take_along_axis(ref["topk_idx"], ri, 1))
        np.testing.assert_allclose(np.take_along_axis(alpha, oi, 1),
                                   np.take_along_axis(ref["alpha"], ri, 1), rtol=TOL_ALPHA, atol=0)
    np.testing.assert_array_equal(out.expert_offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(out.sorted_token_ids.cpu().numpy(), ref["sorted_token_ids"])
    aux = float(out.aux_loss.cpu().numpy()[0])
    if ref["aux"] == 0.0:
        assert aux == 0.0
    else:
        assert abs(aux - ref["aux"]) <= TOL_AUX * abs(ref["aux"]), (aux, ref["aux"])


def sample_rows(N: int, n: int, seed: int = 0) -> np.ndarray:
    """Rows for sampled checks: the first and last tiles' edges plus random rows."""
    if N <= n:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    edge = np.array([0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N - 1, N - 2, N - 65])
    edge = edge[(edge >= 0) & (edge < N)]
    rest = rng.choice(N, size=n - len(edge), replace=False)
    return np.unique(np.concatenate([edge, rest]))


TOL_GRAD = {"fp32": 1e-5, "bf16": 2e-2}   # relative L2 of each gradient (per token / per matrix)
# router-weight gradient, relative L2 per expert row (or the rounding bound of
# dwr_rounding_bound where it is larger, i.e. where d alpha cancels): fp32
# sums over up to 2^14 tokens (measured <= 8.4e-7); bf16 like every other
# bf16 gradient
TOL_DWR = {"fp32": 1e-5, "bf16": 2e-2}


def arr_to_dev(a, dt: str, dev):
    """A storage-dtype numpy array (bf16 bit patterns or float32) on the device."""
    import torch

    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def rel_l2_per_matrix(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over the leading (expert) axis of the Frobenius relative error; a
    matrix whose reference is zero must come out zero."""
    got = got.reshape((-1,) + got.shape[-2:]) if got.ndim >= 2 else got[None]
    ref = ref.reshape(got.shape)
    worst = 0.0
    for g, r in zip(got, ref):
        d = np.linalg.norm(r)
        if d == 0.0:
            if np.abs(g).max(initial=0.0) != 0.0:
                return float("inf")
            continue
        worst = max(worst, float(np.linalg.norm(g - r) / d))
    return worst



def _silu(z):
    return z / (1.0 + np.exp(-z))


def dwr_rounding_bound(f: dict, route: dict, dy64: np.ndarray, k: int, norm_topk_prob: bool,
                       dtype: str, sigmas: float = 5.0) -> np.ndarray:
    """A bound [E, H] on the error of the computed dW_r that comes from the
    rounding of the quantities d alpha is formed from, propagated exactly
    through the (linear) rest of the router's backward: ``sigmas`` times the
    standard deviation of that error under the probabilistic model of
    rounding (independent errors, uniform within the rounding interval).

    d alpha_{t,j} = sum_i dh_i * SiLU(g_i) * u_i with g = W_g x_t, u = W_u x_t,
    dh = W_d^T dy_t (the selected expert's).  Where its terms cancel (few
    tokens per expert), relative errors of g, u, dh of the size of the
    storage rounding become large relative errors of d alpha and of the row
    of dW_r it feeds.  Only the oracle's exact values and the arithmetic's
    unit roundoffs enter: g and u stored in the dtype (a relative error of
    at most u_s = 2^-8 for bf16, 2^-24 for fp32: variance (u_s v)^2 / 3);
    fp32 accumulation of an n-term sum whose terms have magnitude sum S
    (variance n (2^-24 S)^2 / 3); h = SiLU(g) u to first order in the errors
    of g and u.  From d alpha on, the map to dW_r is linear: the
    renormaliser's d p_S (sum_i p_i (d alpha_j - d alpha_i) + 1e-20 d alpha_j)
    / Z^2 (zero for k = 1 up to the 1e-20 term), the softmax's
    d r = p (d p - p . d p) and d W_r = d r^T x; variances add over the
    independent slots and tokens.  Returns sigmas * the standard deviation of
    each element."""
    u_s = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    u32 = 2.0 ** -24
    x = f["x"]
    N, H = x.shape
    E, I = f["Wg"].shape[0], f["Wg"].shape[1]
    p, idx, keep = route["p"], route["topk_idx"], route.get("keep")
    var_dal = np.zeros((N, k))
    for e in range(E):
        tt, jj = np.nonzero(idx == e)
        if keep is not None:
            sel = np.asarray(keep)[tt, jj].astype(bool)
            tt, jj = tt[sel], jj[sel]
        if tt.size == 0:
            continue
        xe, dye = x[tt], dy64[tt]
        Wg, Wu, Wd = f["Wg"][e], f["Wu"][e], f["Wd"][e]
        g, u, d = xe @ Wg.T, xe @ Wu.T, dye @ Wd
        G = np.abs(xe) @ np.abs(Wg).T
        U = np.abs(xe) @ np.abs(Wu).T
        D = np.abs(dye) @ np.abs(Wd)
        sg = 1.0 / (1.0 + np.exp(-g))
        s = g * sg
        ds = sg * (1.0 + g * (1.0 - sg))  # SiLU'
        var_g = ((u_s * g) ** 2 + H * (u32 * G) ** 2) / 3.0
        var_u = ((u_s * u) ** 2 + H * (u32 * U) ** 2) / 3.0
        var_d = H * (u32 * D) ** 2 / 3.0
        var_h = (ds * u) ** 2 * var_g + s ** 2 * var_u
        h = s * u
        var_dal[tt, jj] = ((d ** 2) * var_h + (h ** 2) * var_d).sum(axis=1) + \
            I * (u32 * np.abs(d * h).sum(axis=1)) ** 2 / 3.0
    ps = np.take_along_axis(p, idx, axis=1)                       # [N, k]
    # d p_S = A d alpha per token: A_jj = (sum_{i != j} p_i + 1e-20) / Z^2,
    # A_ji = -p_i / Z^2 (renormalised), A = identity (raw weights)
    if norm_topk_prob:
        Z = ps.sum(axis=1) + 1e-20
        A = np.repeat(-ps[:, None, :] / (Z ** 2)[:, None, None], k, axis=1)  # A[t, j, i]
        diag = (ps.sum(axis=1, keepdims=True) - ps + 1e-20) / (Z ** 2)[:, None]
        ar = np.arange(k)
        A[:, ar, ar] = diag
    else:
        A = np.broadcast_to(np.eye(k), (N, k, k)).copy()
    # d p_te = sum_j [S_tj = e] (A d alpha)_j;  d r = p (d p - p . d p)
    # T[t, e, i]: d r_te per unit d alpha_ti
    P = np.zeros((N, E, k))
    for j in range(k):
        P[np.arange(N), idx[:, j], j] = 1.0
    M = np.einsum("tej,tji->tei", P, A)                           # d p per d alpha
    T = p[:, :, None] * (M - np.einsum("te,tei->ti", p, M)[:, None, :])
    var_dr = np.einsum("tei,ti->te", T ** 2, var_dal)             # [N, E]
    var_dwr = var_dr.T @ (x ** 2)                                 # [E, H]
    return sigmas * np.sqrt(var_dwr)


def check_dwr(got, ref: np.ndarray, bound: np.ndarray, dtype: str) -> None:
    """Every expert row of dW_r within TOL_DWR relative L2, or within the
    rounding bound of dwr_rounding_bound where the arithmetic itself cannot
    give that accuracy (d alpha cancelling); a row whose reference is zero
    must be zero."""
    if not isinstance(got, np.ndarray):
        got = got.detach().double().cpu().numpy()
    for e in range(ref.shape[0]):
        den = np.linalg.norm(ref[e])
        diff = np.linalg.norm(got[e] - ref[e])
        if den < 1e-12:
            assert np.abs(got[e]).max() <= 1e-9, (e, np.abs(got[e]).max())
            continue
        slack = np.linalg.norm(bound[e])
        assert diff <= max(TOL_DWR[dtype] * den, slack), (e, diff / den, slack / den)


def dwr_bound_for(inputs: dict, ref: dict, dy, k: int, norm_topk_prob: bool) -> np.ndarray:
    """dwr_rounding_bound for a parity case: its stored inputs, the oracle's
    backward result (its routing) and the upstream gradient in storage dtype."""
    from oracle.cases import widen
    from workloads import to_f64

    dt = inputs["dtype"]
    return dwr_rounding_bound(widen(inputs), ref["route"], to_f64(dy, dt), k, norm_topk_prob, dt)
