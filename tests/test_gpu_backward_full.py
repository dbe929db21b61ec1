"""Backward parity at the full workload sizes, in the launch configuration the
benchmark times (the same entry points with their default tiles).

The fp64 oracle is compared element by element where it finishes quickly
(the 4096-token top-1 MoE: every gradient), else on exact samples
(oracle.moe_ffn_bwd_sampled / the dense backward on slices): dx on sampled
token rows, and the expert weight gradients on sampled intermediate units,
whose gradients involve only that unit.  Bars as in test_gpu_backward.
"""
import numpy as np
import pytest

from oracle import moe_ffn_bwd_sampled, swiglu_ffn_bwd
from oracle.cases import expected_bwd, make_case, widen
from workloads import get, make_upstream, to_f64
from gpu_util import (TOL_DWR, TOL_GRAD, announce, arr_to_dev, rel_l2_per_matrix,
                      rel_l2_per_token, sample_rows, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def sample_units(I, n=32, seed=1):
    edge = np.array([0, 1, 31, 32, 63, 64, 127, 128, I - 65, I - 64, I - 2, I - 1])
    edge = edge[(edge >= 0) & (edge < I)]
    rest = np.random.default_rng(seed).choice(I, size=n - len(edge), replace=False)
    return np.unique(np.concatenate([edge, rest]))


def to64(t):
    return t.detach().to(__import__("torch").float64).cpu().numpy()


def test_bwd_full_moe_top1(env):
    """4096 tokens, H 768, E 4, k 1: every gradient against the full oracle."""
    torch, dev, tm = env
    w = get("moe_top1_n4096_h768_e4")
    announce(f"moe_ffn_bwd full size {w.name}: inputs and oracle")
    inp = make_case(w)
    dy = make_upstream(inp)
    ref = expected_bwd(w, inp, dy)
    d = to_dev(inp, dev)
    announce("moe_ffn_bwd full size: GPU")
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, w.dtype, dev),
                       w.k, w.coef, norm_topk_prob=w.norm_topk_prob)
    torch.cuda.synchronize()
    assert rel_l2_per_token(y_to_f64(g.dx), ref["dx"]) <= TOL_GRAD[w.dtype]
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(to64(getattr(g, n)), ref[n])
        assert err <= TOL_GRAD[w.dtype], (n, err)
    got = to64(g.dWr)
    for e in range(w.E):
        err = np.linalg.norm(got[e] - ref["dWr"][e]) / np.linalg.norm(ref["dWr"][e])
        assert err <= TOL_DWR[w.dtype], (e, err)


@pytest.mark.parametrize("name", ["moe_top2_skew_n16384_h768_e8", "moe_decode_n32_h2048_e16"])
def test_bwd_full_moe_sampled(env, name):
    """Full-size MoE backward: dx on sampled rows (every row for decode, with
    dW_r), expert weight gradients on sampled units of every expert."""
    torch, dev, tm = env
    w = get(name)
    announce(f"moe_ffn_bwd full size {w.name}: inputs")
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    announce("moe_ffn_bwd full size: GPU")
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, w.dtype, dev),
                       w.k, w.coef, norm_topk_prob=w.norm_topk_prob)
    torch.cuda.synchronize()
    rows = None if w.N <= 64 else sample_rows(w.N, 48)
    units = sample_units(w.I)
    announce("moe_ffn_bwd full size: sampled oracle")
    f = widen(inp)
    ref = moe_ffn_bwd_sampled(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef,
                              to_f64(dy, w.dtype), 1.0, w.norm_topk_prob, rows=rows, units=units)
    r = ref["rows"]
    assert rel_l2_per_token(y_to_f64(g.dx)[r], ref["dx_rows"]) <= TOL_GRAD[w.dtype]
    counts = ref["route"]["counts"]
    for n, gn, sl in (("dWg_u", "dWg", np.s_[:, units]), ("dWu_u", "dWu", np.s_[:, units]),
                      ("dWd_u", "dWd", np.s_[:, :, units])):
        got = to64(getattr(g, gn))[sl]
        err = rel_l2_per_matrix(got, ref[n])
        assert err <= TOL_GRAD[w.dtype], (gn, err, counts.tolist())
    if ref["dWr"] is not None:
        got = to64(g.dWr)
        for e in range(w.E):
            err = np.linalg.norm(got[e] - ref["dWr"][e]) / np.linalg.norm(ref["dWr"][e])
            assert err <= TOL_DWR[w.dtype], (e, err)


def test_bwd_full_dense(env):
    """16384 x 2048 x 6464 dense backward: dx on sampled rows, weight gradients
    on sampled intermediate units (the oracle's backward on those slices)."""
    torch, dev, tm = env
    w = get("dense_bf16_n16384_h2048_i6464")
    announce(f"ffn_swiglu_bwd full size {w.name}: inputs")
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    announce("ffn_swiglu_bwd full size: GPU")
    g = tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, w.dtype, dev))
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 48)
    units = sample_units(w.I)
    announce("ffn_swiglu_bwd full size: sampled oracle")
    f = widen(inp)
    dy64 = to_f64(dy, w.dtype)
    dx_r = swiglu_ffn_bwd(f["x"][rows], f["Wg"], f["Wu"], f["Wd"], dy64[rows])[0]
    _, gWg, gWu, gWd = swiglu_ffn_bwd(f["x"], f["Wg"][units], f["Wu"][units], f["Wd"][:, units], dy64)
    assert rel_l2_per_token(y_to_f64(g.dx)[rows], dx_r) <= TOL_GRAD[w.dtype]
    for got, ref, n in ((to64(g.dWg)[units], gWg, "dWg"), (to64(g.dWu)[units], gWu, "dWu"),
                        (to64(g.dWd)[:, units], gWd, "dWd")):
        err = rel_l2_per_matrix(got, ref)
        assert err <= TOL_GRAD[w.dtype], (n, err)
