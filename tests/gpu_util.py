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
# router-weight gradient, relative L2 per expert row: fp32 sums over up to 2^14
# tokens (~sqrt(N) * 2^-24) times the softmax backward's cancellation; in bf16
# the recomputed g and u are stored in bf16, so d alpha (and dr) carry
# bf16-level error like every other bf16 gradient
TOL_DWR = {"fp32": 1e-4, "bf16": 2e-2}


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



def bf16_of(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest even) and widen them back."""
    from workloads.gen import round_to, to_f64
    return to_f64(round_to(np.asarray(a, dtype=np.float64), "bf16"), "bf16")


def dwr_bf16_h_shift(f: dict, route: dict, dy64: np.ndarray, k: int,
                     norm_topk_prob: bool) -> np.ndarray:
    """The part of the bf16 path's router-weight gradient [E, H] that comes
    from recomputing g and u in bf16: its d alpha_{t,j} is dh_raw . SiLU(g~) u~
    with g~, u~ the bf16-rounded projections (the backward's stored pairs)
    instead of dh_raw . SiLU(g) u.  That change passes linearly through the
    renormalisation (d p_S = d alpha / Z - (d alpha . p_S) / Z^2), the softmax
    (d r = p (d p - p . d p)) and d W_r = d r^T x, so the shift is exact given
    the rounding.  Where d alpha cancels (few tokens per expert), this shift
    dominates the difference to the fp64 oracle."""
    p, idx = route["p"], route["topk_idx"]
    keep = route.get("keep")
    N, E = p.shape
    ddal = np.zeros((N, k))
    for t in range(N):
        for j in range(k):
            if keep is not None and not keep[t, j]:
                continue
            e = idx[t, j]
            g = f["Wg"][e] @ f["x"][t]
            u = f["Wu"][e] @ f["x"][t]
            gb, ub = bf16_of(g), bf16_of(u)
            silu = lambda z: z / (1.0 + np.exp(-z))
            dh_raw = f["Wd"][e].T @ dy64[t]
            ddal[t, j] = dh_raw @ (silu(gb) * ub - silu(g) * u)
    ps = np.take_along_axis(p, idx, axis=1)
    if norm_topk_prob:
        Z = ps.sum(axis=1, keepdims=True) + 1e-20
        dps = ddal / Z - (ddal * ps).sum(axis=1, keepdims=True) / Z ** 2
    else:
        dps = ddal
    dp = np.zeros_like(p)
    np.put_along_axis(dp, idx, dps, axis=1)
    dr = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return dr.T @ f["x"]
