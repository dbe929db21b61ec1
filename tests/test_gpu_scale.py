"""Many experts and large k at production-like sizes (beyond the benchmark
workloads): 64 experts with top-8 / top-6, 32 experts with top-4, 8192-16384
tokens.  These take the router's H-split layout (W_router past 64 KB), the
permutation's multi-block scatter with few router blocks per expert row, and
grouped GEMMs over many small, unequal groups.

The router weights are scaled up (x6 for 64 experts) so that the fp64 top-k
margin of 1e-3 holds for every token after at most a few redraws (with 64
experts and the U(+-1/sqrt(H)) draw many probabilities sit within 1e-3 of
each other).  Routing outputs are compared in full (bit-exact lists, alpha
and aux to 1e-5); y, dx on sampled rows, the expert weight gradients on
sampled units, dW_r in full where every row is taken.  Bars as elsewhere.
"""
import numpy as np
import pytest

from oracle import moe_ffn_bwd_sampled
from oracle.cases import custom_workload, enforce_margin, expected, make_case, widen
from workloads import make_upstream, to_f64
from gpu_util import (TOL_GRAD, TOL_Y, announce, arr_to_dev, check_routing, rel_l2_per_matrix,
                      rel_l2_per_token, run_moe, sample_rows, to_dev, torch_dev, y_to_f64)

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
    rows = sample_rows(N, 256)
    ref = expected(w, inp, rows=rows)
    announce("scale forward: GPU")
    d = to_dev(inp, dev)
    out = run_moe(tm, d, w)
    torch.cuda.synchronize()
    check_routing(out, ref, k, E)
    err = rel_l2_per_token(y_to_f64(out.y)[rows], ref["y"])
    assert err <= TOL_Y[dt], err


def sample_units(I, n=24, seed=3):
    edge = np.array([0, 31, 32, 63, 64, I - 64, I - 1])
    rest = np.random.default_rng(seed).choice(I, size=n - len(edge), replace=False)
    return np.unique(np.concatenate([edge[(edge >= 0) & (edge < I)], rest]))


def test_scale_backward(env):
    """64 experts, top-6, 4096 tokens: dx on sampled rows, weight gradients on
    sampled units of every expert."""
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
    rows = sample_rows(N, 48)
    units = sample_units(I)
    announce("scale backward: sampled oracle")
    f = widen(inp)
    ref = moe_ffn_bwd_sampled(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef,
                              to_f64(dy, "bf16"), 1.0, True, rows=rows, units=units)
    assert rel_l2_per_token(y_to_f64(g.dx)[ref["rows"]], ref["dx_rows"]) <= TOL_GRAD["bf16"]
    to64 = lambda t: t.detach().double().cpu().numpy()
    touched = ref["route"]["counts"] > 0
    for n, gn, sl in (("dWg_u", "dWg", np.s_[:, units]), ("dWu_u", "dWu", np.s_[:, units]),
                      ("dWd_u", "dWd", np.s_[:, :, units])):
        got, want = to64(getattr(g, gn))[sl][touched], ref[n][touched]
        err = rel_l2_per_matrix(got, want)
        assert err <= TOL_GRAD["bf16"], (gn, err)
