"""The down projection split along K (few output tiles, long K: the 100-token
fp32 FFN runs 24 tiles over 76 K slices).  Chunks of K write fp32 partial sums
and a reduce adds them in order and applies the epilogue (alpha, the entry's
destination, the residual, one rounding).  Each case is one the planner splits
(its workspace holds the partials), checked against the oracle; the training
forward takes the same down projection, so its y is the same bits."""
import numpy as np
import pytest

from oracle.cases import custom_workload, expected, make_case
from gpu_util import (TOL_Y, announce, check_routing, rel_l2_per_token, run_dense, run_moe,
                      to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def partial_bytes(w):
    """Workspace bytes beyond the intermediate h (and the slots): the split-K
    partial sums, zero when the planner does not split."""
    from top_moe_layer_amd import _binding as B

    code = B.DTYPE_FP32 if w.dtype == "fp32" else B.DTYPE_BF16
    el = 4 if w.dtype == "fp32" else 2
    if w.kind == "dense":
        return B.raw_ffn_workspace_bytes(w.N, w.H, w.I, code) - w.N * w.I * el
    rows = w.N * w.k
    base = rows * w.I * el + (rows * w.H * el if w.k > 1 else 0)
    return B.raw_moe_workspace_bytes(w.N, w.H, w.I, w.E, w.k, code) - base


DENSE = [(37, 128, 1024, "fp32", False), (100, 256, 2048, "bf16", True),
         (100, 768, 2432, "fp32", True), (3, 64, 512, "bf16", False)]


@pytest.mark.parametrize("N,H,I,dt,res", DENSE)
def test_splitk_dense(env, N, H, I, dt, res):
    torch, dev, tm = env
    w = custom_workload(name="sk_dense", kind="dense", N=N, H=H, I=I, E=1, k=1, coef=0.0,
                        dtype=dt, residual=res, seed=N + H)
    assert partial_bytes(w) >= 2 * N * H * 4  # split in at least two chunks
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"ffn_swiglu_fwd split K: N={N} H={H} I={I} {dt} residual={res}")
    d = to_dev(inp, dev)
    y = run_dense(tm, d)
    # the training forward (keeping g, u) shares the down projection: same bits
    saved = torch.empty(tm.ffn_bwd_workspace_bytes(N, H, I, y.dtype), dtype=torch.uint8,
                        device=dev)
    y2 = tm.ffn_swiglu_fwd(d["x"], d["Wg"], d["Wu"], d["Wd"], residual=d.get("residual"),
                           saved=saved)
    torch.cuda.synchronize()
    err = rel_l2_per_token(y_to_f64(y), ref["y"])
    assert err <= TOL_Y[dt], err
    assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8))


MOE = [  # N, H, I, E, k, dtype, residual, capacity
    (150, 256, 1024, 4, 2, "bf16", True, 0.0),
    (200, 256, 1024, 4, 1, "bf16", True, 1.0),
    (200, 128, 1024, 4, 1, "bf16", False, 0.0),
    (90, 128, 512, 5, 3, "fp32", True, 0.0),
]


@pytest.mark.parametrize("N,H,I,E,k,dt,res,cf", MOE)
def test_splitk_moe(env, N, H, I, E, k, dt, res, cf):
    torch, dev, tm = env
    from oracle import moe_ffn
    from oracle.cases import widen

    w = custom_workload(name="sk_moe", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt,
                        residual=res, seed=N + E + k)
    assert partial_bytes(w) >= 2 * N * k * H * 4
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef,
                  residual=f.get("residual"), capacity_factor=cf)
    announce(f"moe_ffn_fwd split K: N={N} H={H} I={I} E={E} k={k} {dt} residual={res} "
             f"capacity={cf}")
    d = to_dev(inp, dev)
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef,
                         residual=d.get("residual"), capacity_factor=cf)
    torch.cuda.synchronize()
    if cf:
        assert not ref["keep"].all()  # some tokens are dropped
        np.testing.assert_array_equal(out.expert_offsets.cpu().numpy(), ref["kept_offsets"])
    else:
        check_routing(out, ref, k, E)
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y[dt], err
