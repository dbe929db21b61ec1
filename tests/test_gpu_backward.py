"""GPU parity of the backward pass: the HIP path through the C ABI against the
fp64 oracle's gradients on the same seeded inputs and upstream gradient.

Bars (the forward's, carried over; see the tolerance derivation in the design
notes): dx within a max per-token relative L2 error of 1e-5 (fp32) or 2e-2
(bf16 operands, fp32 accumulation); each weight gradient within the same bound
as a relative Frobenius error per expert (an expert with a zero reference
gradient must come out exactly zero); the router-weight gradient (fp32 in both
dtypes) within 1e-4 per expert row on the fp32 path and 2e-2 on the bf16 path
(where the recomputed g, u feeding d alpha are bf16).  Inputs keep the top-k margin of 1e-3, so
the routing the backward recomputes is the oracle's.
"""
import numpy as np
import pytest

from oracle.cases import custom_workload, expected_bwd, make_case
from workloads import make_upstream
from gpu_util import (TOL_GRAD, announce, arr_to_dev, check_dwr, dwr_bound_for,
                      rel_l2_per_matrix, rel_l2_per_token, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def dense_grads(tm, d, dy):
    return tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], dy)


def moe_grads(tm, d, dy, w, aux_grad=1.0):
    return tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dy, w.k, w.coef,
                          aux_grad=aux_grad, norm_topk_prob=w.norm_topk_prob)


def check_weight_grads(g, ref, dt, names=("dWg", "dWu", "dWd")):
    for n in names:
        err = rel_l2_per_matrix(y_to_f64(getattr(g, n)), ref[n])
        assert err <= TOL_GRAD[dt], (n, err)


# ------------------------------------------------------------------ dense
DENSE_BWD = [(1, 64, 64), (100, 128, 192), (300, 256, 320), (513, 192, 448)]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,H,I", DENSE_BWD)
def test_dense_bwd(env, N, H, I, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"dbwd_{N}_{H}_{I}", kind="dense", N=N, H=H, I=I, E=1, k=1,
                        coef=0.0, dtype=dt, seed=3 * N + H + I)
    inp = make_case(w)
    dy = make_upstream(inp)
    ref = expected_bwd(w, inp, dy)
    announce(f"ffn_swiglu_bwd N={N} H={H} I={I} {dt}")
    g = dense_grads(tm, to_dev(inp, dev), arr_to_dev(dy, dt, dev))
    torch.cuda.synchronize()
    err = rel_l2_per_token(y_to_f64(g.dx), ref["dx"])
    assert err <= TOL_GRAD[dt], ("dx", err)
    check_weight_grads(g, ref, dt)


def test_dense_bwd_empty(env):
    torch, dev, tm = env
    announce("ffn_swiglu_bwd N=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = lambda *s: torch.randn(*s, device=dev).to(torch.bfloat16)
    g = tm.ffn_swiglu_bwd(x, W(128, 64), W(128, 64), W(64, 128), x)
    torch.cuda.synchronize()
    assert g.dx.shape == (0, 64)
    for t in (g.dWg, g.dWu, g.dWd):
        assert t.abs().max().item() == 0.0


# -------------------------------------------------------------------- moe
MOE_BWD = [
    # N, H, I, E, k, coef, norm_topk_prob, dtype
    (300, 128, 192, 8, 2, 0.01, True, "bf16"),
    (300, 128, 192, 8, 2, 0.01, False, "bf16"),
    (257, 64, 128, 4, 1, 0.01, True, "bf16"),
    (257, 64, 128, 4, 1, 0.0, True, "bf16"),
    (200, 64, 64, 4, 4, 0.02, True, "bf16"),
    (129, 128, 64, 3, 1, 0.05, False, "bf16"),
    (1000, 64, 64, 16, 2, 0.01, True, "bf16"),
    (1, 64, 64, 4, 1, 0.01, True, "bf16"),
    (150, 64, 128, 8, 2, 0.01, True, "fp32"),
    (100, 64, 64, 4, 3, 0.01, False, "fp32"),
]


@pytest.mark.parametrize("N,H,I,E,k,coef,norm,dt", MOE_BWD)
def test_moe_bwd(env, N, H, I, E, k, coef, norm, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"mbwd_{N}_{H}_{I}_{E}_{k}", N=N, H=H, I=I, E=E, k=k, coef=coef,
                        dtype=dt, norm_topk_prob=norm, seed=N + 7 * E + k)
    inp = make_case(w)
    dy = make_upstream(inp)
    ref = expected_bwd(w, inp, dy, daux=1.5)
    announce(f"moe_ffn_bwd N={N} H={H} I={I} E={E} k={k} coef={coef} norm={norm} {dt}")
    g = moe_grads(tm, to_dev(inp, dev), arr_to_dev(dy, dt, dev), w, aux_grad=1.5)
    torch.cuda.synchronize()
    err = rel_l2_per_token(y_to_f64(g.dx), ref["dx"])
    assert err <= TOL_GRAD[dt], ("dx", err)
    check_weight_grads(g, ref, dt)
    check_dwr(g.dWr, ref["dWr"], dwr_bound_for(inp, ref, dy, k, norm), dt)


def test_moe_bwd_empty_experts(env):
    """Per-expert logit offsets large enough to leave experts without tokens:
    their weight gradients must be exactly zero."""
    torch, dev, tm = env
    w = custom_workload(name="mbwd_skew", N=300, H=128, I=128, E=8, k=2, coef=0.01,
                        bias_std=1.5, bias_scale=1.0, seed=11)
    inp = make_case(w)
    dy = make_upstream(inp)
    ref = expected_bwd(w, inp, dy)
    counts = np.bincount(ref["route"]["topk_idx"].ravel(), minlength=w.E)
    assert (counts == 0).any(), counts
    announce(f"moe_ffn_bwd skewed, expert counts {counts.tolist()}")
    g = moe_grads(tm, to_dev(inp, dev), arr_to_dev(dy, "bf16", dev), w)
    torch.cuda.synchronize()
    for n in ("dWg", "dWu", "dWd"):
        got = getattr(g, n).float().cpu().numpy()
        for e in np.nonzero(counts == 0)[0]:
            assert np.abs(got[e]).max() == 0.0, (n, e)
    err = rel_l2_per_token(y_to_f64(g.dx), ref["dx"])
    assert err <= TOL_GRAD["bf16"], ("dx", err)
    check_weight_grads(g, ref, "bf16")
    check_dwr(g.dWr, ref["dWr"], dwr_bound_for(inp, ref, dy, w.k, w.norm_topk_prob), "bf16")


def test_moe_bwd_empty_batch(env):
    torch, dev, tm = env
    announce("moe_ffn_bwd N=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = lambda *s: torch.randn(*s, device=dev).to(torch.bfloat16)
    Wr = torch.randn(4, 64, device=dev)
    g = tm.moe_ffn_bwd(x, Wr, W(4, 128, 64), W(4, 128, 64), W(4, 64, 128), x, 2, 0.01)
    torch.cuda.synchronize()
    for t in (g.dWr, g.dWg, g.dWu, g.dWd):
        assert t.abs().max().item() == 0.0


def test_moe_bwd_deterministic(env):
    torch, dev, tm = env
    w = custom_workload(name="mbwd_det", N=777, H=128, I=192, E=8, k=2, coef=0.01, seed=5)
    inp = make_case(w)
    dy = make_upstream(inp)
    d = to_dev(inp, dev)
    dyd = arr_to_dev(dy, "bf16", dev)
    announce("moe_ffn_bwd twice, bitwise")
    a = moe_grads(tm, d, dyd, w)
    b = moe_grads(tm, d, dyd, w)
    torch.cuda.synchronize()
    for n in ("dx", "dWr", "dWg", "dWu", "dWd"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
