"""The autograd bindings inside a PyTorch graph: loss = sum(dy * y) + daux *
aux_loss + dz * z_loss, backpropagated by torch, against the oracle's
gradients (bars as in test_gpu_backward)."""
import numpy as np
import pytest

from oracle import moe_ffn_bwd, swiglu_ffn_bwd
from oracle.cases import custom_workload, make_case, widen
from workloads import make_upstream, to_f64
from gpu_util import (TOL_GRAD, check_dwr, dwr_bound_for, announce, arr_to_dev, rel_l2_per_matrix,
                      rel_l2_per_token, to_dev, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def grads_of(d, names):
    return {n: d[n].grad.detach().double().cpu().numpy() for n in names}


def test_autograd_dense(env):
    torch, dev, tm = env
    w = custom_workload(name="ag_dense", kind="dense", N=200, H=128, I=192, E=1, k=1, coef=0.0,
                        seed=21)
    inp = make_case(w)
    dy = make_upstream(inp)
    d = {n: t.requires_grad_() for n, t in to_dev(inp, dev).items()}
    dyd = arr_to_dev(dy, "bf16", dev)
    announce("autograd swiglu_ffn N=200")
    y = tm.swiglu_ffn(d["x"], d["Wg"], d["Wu"], d["Wd"])
    (y.float() * dyd.float()).sum().backward()
    torch.cuda.synchronize()
    f = widen(inp)
    dx, dWg, dWu, dWd = swiglu_ffn_bwd(f["x"], f["Wg"], f["Wu"], f["Wd"], to_f64(dy, "bf16"))
    g = grads_of(d, ("x", "Wg", "Wu", "Wd"))
    assert rel_l2_per_token(g["x"], dx) <= TOL_GRAD["bf16"]
    for n, ref in (("Wg", dWg), ("Wu", dWu), ("Wd", dWd)):
        assert rel_l2_per_matrix(g[n], ref) <= TOL_GRAD["bf16"], n


def test_autograd_moe_with_losses(env):
    torch, dev, tm = env
    w = custom_workload(name="ag_moe", N=300, H=128, I=128, E=8, k=2, coef=0.01, seed=22)
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    for n in ("x", "Wg", "Wu", "Wd", "Wr"):
        d[n].requires_grad_()
    dyd = arr_to_dev(dy, "bf16", dev)
    announce("autograd moe_ffn N=300 E=8 k=2 with aux and z losses")
    y, aux, z, idx, alpha = tm.moe_ffn(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef,
                                       z_coef=0.001)
    loss = (y.float() * dyd.float()).sum() + 1.5 * aux.sum() + 0.5 * z.sum()
    loss.backward()
    torch.cuda.synchronize()
    f = widen(inp)
    ref = moe_ffn_bwd(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef, to_f64(dy, "bf16"),
                      1.5, True, z_coef=0.001, dz=0.5)
    g = grads_of(d, ("x", "Wr", "Wg", "Wu", "Wd"))
    assert rel_l2_per_token(g["x"], ref["dx"]) <= TOL_GRAD["bf16"]
    for n, r in (("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd")):
        assert rel_l2_per_matrix(g[n], ref[r]) <= TOL_GRAD["bf16"], n
    check_dwr(g["Wr"], ref["dWr"], dwr_bound_for(inp, ref, dy, w.k, True), "bf16")
