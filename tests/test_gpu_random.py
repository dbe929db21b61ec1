"""Seeded random sweep over the shape and option space: 24 forward and 12
backward cases with shapes, expert counts, k, dtype, residual, the raw
top-k weights, z-loss and capacity drawn at random (H and I multiples of 64,
as the ABI requires), each checked against the oracle to the bars of the
fixed-shape tests (dW_r: the relative bar plus an a-priori rounding bound,
which is what remains where few tokens per expert leave d alpha badly
conditioned).  The draw is fixed (seed below), so a failure names a
reproducible case."""
import numpy as np
import pytest

from oracle import moe_ffn, moe_ffn_bwd
from oracle.cases import custom_workload, expected, make_case, widen
from workloads import make_upstream, to_f64
from gpu_util import (TOL_GRAD, TOL_Y, announce, arr_to_dev, check_dwr, check_routing,
                      dwr_bound_for, rel_l2_per_matrix, rel_l2_per_token, to_dev, torch_dev,
                      y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def draw(n, seed, bwd=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 6, 7, 8, 12, 16, 24]))
        k = int(rng.integers(1, min(E, 6) + 1))
        out.append(dict(
            i=i,
            N=int(rng.choice([1, 3, 17, 64, 65, 127, 255, 300, 511, 777, 1500])),
            H=64 * int(rng.integers(1, 5 if bwd else 9)),
            I=64 * int(rng.integers(1, 6 if bwd else 11)),
            E=E, k=k,
            dt=str(rng.choice(["bf16", "bf16", "fp32"])),
            res=bool(rng.random() < 0.3) and not bwd,
            norm=bool(rng.random() < 0.8),
            zc=float(rng.choice([0.0, 0.0, 0.003])),
            cf=float(rng.choice([0.0, 0.0, 0.0, 1.0, 1.5])) if k < E else 0.0,
        ))
    return out


FWD = draw(24, 20261202)
BWD = draw(12, 777, bwd=True)


def name(c):
    return (f"{c['i']}-N{c['N']}-H{c['H']}-I{c['I']}-E{c['E']}-k{c['k']}-{c['dt']}"
            f"{'-res' if c['res'] else ''}{'' if c['norm'] else '-raw'}"
            f"{'-z' if c['zc'] else ''}{'-cap' if c['cf'] else ''}")


@pytest.mark.parametrize("c", FWD, ids=name)
def test_random_forward(env, c):
    torch, dev, tm = env
    w = custom_workload(name="rnd", N=c["N"], H=c["H"], I=c["I"], E=c["E"], k=c["k"], coef=0.01,
                        dtype=c["dt"], residual=c["res"], norm_topk_prob=c["norm"],
                        seed=1000 + c["i"])
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef,
                  residual=f.get("residual"), norm_topk_prob=c["norm"], z_coef=c["zc"],
                  capacity_factor=c["cf"])
    announce(f"random forward {name(c)}")
    d = to_dev(inp, dev)
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef,
                         residual=d.get("residual"), norm_topk_prob=c["norm"], z_coef=c["zc"],
                         capacity_factor=c["cf"])
    torch.cuda.synchronize()
    if c["cf"]:  # the lists then hold the kept entries
        ref = dict(ref, offsets=ref["kept_offsets"])
        nk = len(ref["kept_sorted_token_ids"])
        ids = out.sorted_token_ids.cpu().numpy()
        np.testing.assert_array_equal(ids[:nk], ref["kept_sorted_token_ids"])
        assert (ids[nk:] == -1).all()
        np.testing.assert_array_equal(out.expert_offsets.cpu().numpy(), ref["kept_offsets"])
        np.testing.assert_array_equal(out.topk_idx.cpu().numpy(), ref["topk_idx"])
        np.testing.assert_allclose(out.alpha.cpu().numpy(), ref["alpha"], rtol=1e-5, atol=0)
        aux = float(out.aux_loss.cpu()[0])
        assert abs(aux - ref["aux"]) <= 1e-5 * abs(ref["aux"]), (aux, ref["aux"])
    else:
        check_routing(out, ref, w.k, w.E, exact_order=w.k < w.E)
    if c["zc"]:
        z = float(out.z_loss.cpu()[0])
        assert abs(z - ref["z_loss"]) <= 1e-5 * ref["z_loss"], (z, ref["z_loss"])
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y[c["dt"]], err


@pytest.mark.parametrize("c", BWD, ids=name)
def test_random_backward(env, c):
    torch, dev, tm = env
    w = custom_workload(name="rndb", N=c["N"], H=c["H"], I=c["I"], E=c["E"], k=c["k"], coef=0.01,
                        dtype=c["dt"], norm_topk_prob=c["norm"], seed=2000 + c["i"])
    inp = make_case(w)
    dy = make_upstream(inp)
    f = widen(inp)
    ref = moe_ffn_bwd(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], w.k, w.coef,
                      to_f64(dy, c["dt"]), 0.7, c["norm"], z_coef=c["zc"], dz=1.3,
                      capacity_factor=c["cf"])
    announce(f"random backward {name(c)}")
    d = to_dev(inp, dev)
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, c["dt"], dev),
                       w.k, w.coef, aux_grad=0.7, norm_topk_prob=c["norm"], z_coef=c["zc"],
                       z_grad=1.3, capacity_factor=c["cf"])
    torch.cuda.synchronize()
    assert rel_l2_per_token(y_to_f64(g.dx), ref["dx"]) <= TOL_GRAD[c["dt"]]
    to64 = lambda t: t.detach().double().cpu().numpy()
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(to64(getattr(g, n)), ref[n])
        assert err <= TOL_GRAD[c["dt"]], (n, err)
    # dW_r: the relative bar plus the a-priori rounding bound (which is what
    # remains where d alpha cancels, with few tokens per expert)
    check_dwr(to64(g.dWr), ref["dWr"], dwr_bound_for(inp, ref, dy, w.k, c["norm"]), c["dt"])
