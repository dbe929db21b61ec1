"""Parity cases: seeded inputs plus the oracle's expected outputs.

TEST INFRASTRUCTURE ONLY.  Builds inputs with ``workloads`` and, for MoE cases,
redraws token rows whose top-k decision is too close to call: in float64 from
the stored inputs, every adjacent gap among the first min(k+1, E) sorted
probabilities must be at least ``MARGIN`` (ties are otherwise decided by
rounding, and no two correct implementations need agree on them).  For k == E
the selected set is all experts, so no margin is imposed.
"""
from __future__ import annotations

import numpy as np

import workloads
from workloads import Workload, make_inputs, redraw_token_rows, to_f64

from .ffn_moe import router_probs, moe_ffn, dense_ffn, moe_route, swiglu_ffn_bwd, moe_ffn_bwd

MARGIN = 1e-3
MAX_REDRAWS = 64


def widen(inputs: dict) -> dict:
    """Float64 views of the stored tensors (exact widening)."""
    dt = inputs["dtype"]
    out = {"x": to_f64(inputs["x"], dt)}
    for n in ("Wg", "Wu", "Wd", "residual"):
        if n in inputs:
            out[n] = to_f64(inputs[n], dt)
    if "Wr" in inputs:
        out["Wr"] = inputs["Wr"].astype(np.float64)
    return out


def small_margin_rows(x64, Wr64, k, margin=MARGIN):
    """Token rows whose first min(k+1, E) sorted probabilities are not all
    separated by at least ``margin``."""
    E = Wr64.shape[0]
    if k >= E:
        return np.zeros(0, dtype=np.int64)
    p = router_probs(x64, Wr64)
    ps = -np.sort(-p, axis=1)[:, : min(k + 1, E)]
    gaps = ps[:, :-1] - ps[:, 1:]
    return np.nonzero((gaps < margin).any(axis=1))[0]


def enforce_margin(inputs: dict, k: int, margin=MARGIN) -> dict:
    """Redraw failing token rows in place until every row clears the margin."""
    Wr64 = inputs["Wr"].astype(np.float64)
    dt = inputs["dtype"]
    bad = small_margin_rows(to_f64(inputs["x"], dt), Wr64, k, margin)
    total = int(bad.size)
    attempt = 0
    while bad.size:
        if attempt >= MAX_REDRAWS:
            raise RuntimeError(f"{bad.size} token rows still inside the top-k margin")
        redraw_token_rows(inputs, bad, attempt)
        x_bad = to_f64(inputs["x"][bad], dt)
        still = small_margin_rows(x_bad, Wr64, k, margin)
        bad = bad[still]
        attempt += 1
    inputs["redrawn_rows"] = total
    return inputs


def make_case(w: Workload, seed=None, N=None, margin=True) -> dict:
    """Inputs for ``w`` (margin-enforced for MoE)."""
    inp = make_inputs(w, seed=seed, N=N)
    if w.kind == "moe" and margin:
        enforce_margin(inp, w.k)
    return inp


def expected(w: Workload, inputs: dict, rows=None) -> dict:
    """Oracle outputs for ``inputs``; ``rows`` restricts y to those tokens."""
    f = widen(inputs)
    res = f.get("residual")
    if w.kind == "dense":
        return {"y": dense_ffn(f["x"], f["Wg"], f["Wu"], f["Wd"], rows=rows, residual=res),
                "rows": np.arange(f["x"].shape[0]) if rows is None else np.asarray(rows)}
    return moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef, rows=rows,
                   residual=res, norm_topk_prob=w.norm_topk_prob)


def expected_route(w: Workload, inputs: dict) -> dict:
    f = widen(inputs)
    return moe_route(f["x"], f["Wr"], w.k, w.coef, w.norm_topk_prob)


def expected_bwd(w: Workload, inputs: dict, dy, daux: float = 1.0) -> dict:
    """Oracle gradients for ``inputs`` and the upstream gradient ``dy``
    (storage dtype): dx, dWg, dWu, dWd (+ dWr and the routing for MoE)."""
    f = widen(inputs)
    dy64 = to_f64(dy, inputs["dtype"])
    if w.kind == "dense":
        dx, dWg, dWu, dWd = swiglu_ffn_bwd(f["x"], f["Wg"], f["Wu"], f["Wd"], dy64)
        return {"dx": dx, "dWg": dWg, "dWu": dWu, "dWd": dWd}
    return moe_ffn_bwd(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef, dy64, daux,
                       w.norm_topk_prob)


def custom_workload(**kw) -> Workload:
    """Ad-hoc workload for edge-case tests (random small shapes)."""
    base = dict(name="custom", kind="moe", N=16, H=64, I=64, E=4, k=1, coef=0.01, dtype="bf16")
    base.update(kw)
    return Workload(**base)


__all__ = [
    "MARGIN", "widen", "small_margin_rows", "enforce_margin", "make_case",
    "expected", "expected_route", "expected_bwd", "custom_workload", "workloads",
]
