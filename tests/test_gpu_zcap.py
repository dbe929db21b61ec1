"""GPU parity of the router z-loss and the expert capacity (token dropping),
forward and backward, against the oracle's readings of them (standard forms;
the pages only name both).

Bars: z_loss within 1e-5 relative; under a capacity the kept offsets and the
kept token lists (ending in -1) bit-exact, topk_idx / alpha / aux unchanged
(the router's choices, before dropping), y and the gradients within the bars
of the plain path (y and dx per token: 1e-5 fp32 / 2e-2 bf16; weight
gradients per expert; dW_r per expert row 1e-4 fp32 / 2e-2 bf16).
"""
import numpy as np
import pytest

from oracle import moe_ffn, moe_ffn_bwd
from oracle.cases import custom_workload, make_case, widen
from workloads import make_upstream, to_f64
from gpu_util import (TOL_GRAD, check_dwr, dwr_bound_for, TOL_Y, announce, arr_to_dev, rel_l2_per_matrix,
                      rel_l2_per_token, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def to64(t):
    return t.detach().double().cpu().numpy()


FWD = [
    # N, H, I, E, k, z_coef, capacity_factor, residual, dtype
    (300, 128, 128, 8, 2, 0.001, 0.0, False, "bf16"),    # z-loss, LDS-mode router
    (100, 128, 64, 4, 1, 0.01, 0.0, False, "bf16"),      # z-loss, split-mode router
    (300, 128, 128, 8, 2, 0.0, 1.0, False, "bf16"),      # capacity, k = 2
    (257, 64, 128, 4, 1, 0.002, 0.8, True, "bf16"),      # capacity, k = 1, residual
    (200, 64, 64, 4, 2, 0.01, 0.5, True, "fp32"),
    (1000, 64, 64, 16, 2, 0.0, 1.1, False, "bf16"),
]


@pytest.mark.parametrize("N,H,I,E,k,zc,cf,res,dt", FWD)
def test_zcap_forward(env, N, H, I, E, k, zc, cf, res, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"zcap_{N}_{E}_{k}", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt,
                        residual=res, seed=N + 13 * E + k)
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef,
                  residual=f.get("residual"), z_coef=zc, capacity_factor=cf)
    announce(f"moe_ffn_fwd z_coef={zc} capacity={cf} N={N} E={E} k={k} {dt}")
    d = to_dev(inp, dev)
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef,
                         residual=d.get("residual"), z_coef=zc, capacity_factor=cf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.topk_idx.cpu().numpy(), ref["topk_idx"])
    np.testing.assert_allclose(out.alpha.cpu().numpy(), ref["alpha"], rtol=1e-5, atol=0)
    assert abs(float(out.aux_loss.cpu()[0]) - ref["aux"]) <= 1e-5 * ref["aux"]
    if zc:
        z = float(out.z_loss.cpu()[0])
        assert abs(z - ref["z_loss"]) <= 1e-5 * ref["z_loss"], (z, ref["z_loss"])
    np.testing.assert_array_equal(out.expert_offsets.cpu().numpy(), ref["kept_offsets"])
    ids = out.sorted_token_ids.cpu().numpy()
    nk = len(ref["kept_sorted_token_ids"])
    np.testing.assert_array_equal(ids[:nk], ref["kept_sorted_token_ids"])
    assert (ids[nk:] == -1).all()
    if cf:
        assert not ref["keep"].all(), "the case drops something"
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y[dt], err


BWD = [
    # N, H, I, E, k, z_coef, capacity_factor, norm, dtype
    (300, 128, 192, 8, 2, 0.001, 0.0, True, "bf16"),
    (300, 128, 192, 8, 2, 0.0, 0.9, True, "bf16"),
    (257, 64, 128, 4, 1, 0.01, 0.6, True, "bf16"),
    (200, 64, 128, 8, 2, 0.005, 0.7, False, "fp32"),
    (150, 64, 64, 4, 1, 0.02, 0.0, True, "fp32"),
]


@pytest.mark.parametrize("N,H,I,E,k,zc,cf,norm,dt", BWD)
def test_zcap_backward(env, N, H, I, E, k, zc, cf, norm, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"zcapb_{N}_{E}_{k}", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt,
                        norm_topk_prob=norm, seed=2 * N + E + k)
    inp = make_case(w)
    dy = make_upstream(inp)
    f = widen(inp)
    ref = moe_ffn_bwd(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef, to_f64(dy, dt), 1.2,
                      norm, z_coef=zc, dz=0.8, capacity_factor=cf)
    announce(f"moe_ffn_bwd z_coef={zc} capacity={cf} N={N} E={E} k={k} {dt}")
    d = to_dev(inp, dev)
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, dt, dev), k,
                       w.coef, aux_grad=1.2, norm_topk_prob=norm, z_coef=zc, z_grad=0.8,
                       capacity_factor=cf)
    torch.cuda.synchronize()
    if cf:
        assert not ref["route"]["keep"].all()
    err = rel_l2_per_token(y_to_f64(g.dx), ref["dx"])
    assert err <= TOL_GRAD[dt], ("dx", err)
    for n in ("dWg", "dWu", "dWd"):
        e = rel_l2_per_matrix(to64(getattr(g, n)), ref[n])
        assert e <= TOL_GRAD[dt], (n, e)
    check_dwr(to64(g.dWr), ref["dWr"], dwr_bound_for(inp, ref, dy, k, norm), dt)
