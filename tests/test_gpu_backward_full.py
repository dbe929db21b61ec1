"""Backward parity at the full workload sizes, in the launch configuration the
benchmark times (the same entry points with their default tiles).

Every gradient is compared with the fp64 oracle's full backward: dx on every
token row, every expert's dW_g, dW_u and dW_d, dW_r per expert row.  Bars as
in test_gpu_backward (dW_r: relative bar plus the a-priori rounding bound).
"""
import numpy as np
import pytest

from oracle.cases import expected_bwd, make_case
from workloads import get, make_upstream
from gpu_util import (TOL_GRAD, announce, arr_to_dev, check_dwr, dwr_bound_for,
                      rel_l2_per_matrix, rel_l2_per_token, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def to64(t):
    return t.detach().to(__import__("torch").float64).cpu().numpy()


MOE_FULL = ["moe_top1_n4096_h768_e4", "moe_top2_skew_n16384_h768_e8",
            "moe_top2_skew_literal_n16384_h768_e8", "moe_decode_n32_h2048_e16"]


@pytest.mark.parametrize("name", MOE_FULL)
def test_bwd_full_moe(env, name):
    torch, dev, tm = env
    w = get(name)
    announce(f"moe_ffn_bwd full size {w.name}: inputs")
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    announce(f"moe_ffn_bwd full size {w.name}: GPU")
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, w.dtype, dev),
                       w.k, w.coef, norm_topk_prob=w.norm_topk_prob)
    torch.cuda.synchronize()
    got = {n: to64(getattr(g, n)) for n in ("dx", "dWr", "dWg", "dWu", "dWd")}
    del g
    announce(f"moe_ffn_bwd full size {w.name}: oracle")
    ref = expected_bwd(w, inp, dy)
    err = rel_l2_per_token(got["dx"], ref["dx"])
    print(f"[gpu] {w.name} dx max per-token rel L2 {err:.3e}", flush=True)
    assert err <= TOL_GRAD[w.dtype], err
    counts = ref["route"]["counts"]
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(got[n], ref[n])
        assert err <= TOL_GRAD[w.dtype], (n, err, counts.tolist())
    check_dwr(got["dWr"], ref["dWr"], dwr_bound_for(inp, ref, dy, w.k, w.norm_topk_prob),
              w.dtype)


def test_bwd_full_dense(env):
    """16384 x 2048 x 6464 dense backward: every gradient."""
    torch, dev, tm = env
    w = get("dense_bf16_n16384_h2048_i6464")
    announce(f"ffn_swiglu_bwd full size {w.name}: inputs")
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    announce(f"ffn_swiglu_bwd full size {w.name}: GPU")
    g = tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, w.dtype, dev))
    torch.cuda.synchronize()
    got = {n: to64(getattr(g, n)) for n in ("dx", "dWg", "dWu", "dWd")}
    del g, d
    announce(f"ffn_swiglu_bwd full size {w.name}: oracle")
    ref = expected_bwd(w, inp, dy)
    err = rel_l2_per_token(got["dx"], ref["dx"])
    print(f"[gpu] {w.name} dx max per-token rel L2 {err:.3e}", flush=True)
    assert err <= TOL_GRAD[w.dtype], err
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(got[n], ref[n])
        assert err <= TOL_GRAD[w.dtype], (n, err)
