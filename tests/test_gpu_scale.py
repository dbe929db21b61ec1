"""Many experts and large k at production-like sizes (beyond the benchmark
workloads): 64 experts with top-8 / top-6, 32 experts with top-4, 8192-16384
tokens.  These take the router's H-split layout (W_router past 64 KB), the
permutation's multi-block scatter with few router blocks per expert row, and
grouped GEMMs over many small, unequal groups.

The router weights are scaled up (x6 for 64 experts) so that the fp64 top-k
margin of 1e-3 holds for every token after at most a few redraws (with 64
experts and the U(+-1/sqrt(H)) draw many probabilities sit within 1e-3 of
each other).  Everything is compared in full: routing outputs (bit-exact
lists, alpha and aux to 1e-5), y and dx on every token row, every expert's
weight gradients.  Bars as elsewhere.
"""
import numpy as np
import pytest

from oracle.cases import custom_workload, enforce_margin, expected, expected_bwd, make_case
from workloads import make_upstream
from gpu_util import (TOL_GRAD, TOL_Y, announce, arr_to_dev, check_routing, rel_l2_per_matrix,
                      rel_l2_per_token, run_moe, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def scaled_case(w, scale):
    inp = make_case(w, margin=False)
    inp["Wr"] = (np.asarray(inp["Wr"], dtype=np.float64) * scale).astype(np.float32)
    enforce_margin(inp, w.k)
    return inp


SCALE_FWD = [
    # N, H, I, E, k, router scale, dtype
    (8192, 1024, 512, 64, 8, 6.0, "bf16"),
    (16384, 1024, 1024, 32, 4, 1.0, "bf16"),
    (4096, 512, 256, 64, 6, 6.0, "fp32"),
]


@pytest.mark.parametrize("N,H,I,E,k,sc,dt", SCALE_FWD)
def test_scale_forward(env, N, H, I, E, k, sc, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"scale_{E}x{k}", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt,
                        seed=E + k)
    announce(f"scale forward N={N} H={H} I={I} E={E} k={k} {dt}: inputs (margin redraws)")
    inp = scaled_case(w, sc)
    ref = expected(w, inp)
    announce("scale forward: GPU")
    d = to_dev(inp, dev)
    out = run_moe(tm, d, w)
    torch.cuda.synchronize()
    check_routing(out, ref, k, E)
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y[dt], err


def test_scale_backward(env):
    """64 experts, top-6, 4096 tokens: every gradient against the oracle's
    full backward (dx per token; dW_g, dW_u, dW_d per expert)."""
    torch, dev, tm = env
    N, H, I, E, k = 4096, 512, 256, 64, 6
    w = custom_workload(name="scale_bwd", N=N, H=H, I=I, E=E, k=k, coef=0.01, seed=71)
    announce(f"scale backward N={N} H={H} I={I} E={E} k={k}: inputs")
    inp = scaled_case(w, 6.0)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    announce("scale backward: GPU")
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, "bf16", dev),
                       k, w.coef)
    torch.cuda.synchronize()
    announce("scale backward: oracle")
    ref = expected_bwd(w, inp, dy)
    assert rel_l2_per_token(y_to_f64(g.dx), ref["dx"]) <= TOL_GRAD["bf16"]
    to64 = lambda t: t.detach().double().cpu().numpy()
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(to64(getattr(g, n)), ref[n])
        assert err <= TOL_GRAD["bf16"], (n, err)
