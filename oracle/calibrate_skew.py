"""Calibrate the logit-offset scale of the skewed top-2 MoE workload.

TEST INFRASTRUCTURE ONLY.  The workload asks for per-expert logit offsets drawn
from N(0, 1.5) "so that per-expert loads differ by up to about 10x".  With
uniform-init router weights the logit spread is only ~0.58, so unscaled
offsets empty several experts; this script finds the single scale s applied to
the drawn offsets that makes max_e c_e / min_e c_e closest to 10 on the seed-0
inputs (bisection on log-ratio, which grows monotonically with s here), using
only the oracle's routing.

    python -m oracle.calibrate_skew          # prints s and the per-expert loads
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

from workloads import get, make_inputs, to_f64
from .ffn_moe import router_probs, topk_canonical, expert_lists


def load_ratio(w, s):
    wk = dataclasses.replace(w, bias_scale=s)
    inp = make_inputs(wk)
    p = router_probs(to_f64(inp["x"], inp["dtype"]), inp["Wr"].astype(np.float64))
    counts, _, _ = expert_lists(topk_canonical(p, wk.k), wk.E)
    return (counts.max() / max(counts.min(), 1)), counts


def calibrate(name="moe_skew", target=10.0, lo=0.0, hi=1.0, iters=18):
    w = get(name)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r, _ = load_ratio(w, mid)
        if r < target:
            lo = mid
        else:
            hi = mid
    s = round(0.5 * (lo + hi), 3)
    r, counts = load_ratio(w, s)
    return s, r, counts


if __name__ == "__main__":
    s, r, counts = calibrate()
    print(f"bias_scale={s} max/min={r:.2f} counts={counts.tolist()}")
    sys.exit(0)
