"""Every instantiated GEMM launch shape (block tile, wavefront grid, LDS row
bytes, ring depth), forced through the planner's override
(topmoe_set_tile_override), against the fp64 oracle on dense and MoE cases
with ragged tails."""
import pytest

from oracle.cases import custom_workload, expected, make_case
from gpu_util import TOL_Y, announce, check_routing, rel_l2_per_token, run_dense, run_moe, to_dev, torch_dev, y_to_f64

pytestmark = pytest.mark.gpu

BF16_SHAPES = [
    "128x64x2x2x128x2", "128x64x2x2x128x3", "128x64x2x2x64x4",
    "128x128x2x2x128x2", "128x128x2x2x128x3", "128x128x2x2x64x4",
    "64x64x2x2x128x3", "64x64x2x2x128x4",
    "256x128x4x2x64x4", "256x128x4x2x64x3", "256x256x4x2x64x4",
    "128x128x2x4x64x4", "256x128x4x2x128x2", "128x128x2x4x128x3",
    "128x128x2x4x128x4", "256x64x4x2x128x3", "256x128x4x2x128x3",
    "64x128x2x4x128x3", "256x256x4x2x128x2",
]
# shapes whose LDS ring does not fit for the gate/up projection (two weight panels)
GATEUP_TOO_BIG = {"128x128x2x2x128x3", "256x256x4x2x64x4", "128x128x2x4x128x4",
                  "256x128x4x2x128x3", "256x256x4x2x128x2"}


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


@pytest.fixture
def shape_env():
    from top_moe_layer_amd import _binding as B

    yield B.set_tile_override
    for g in B.TILE_SLOTS:
        B.set_tile_override(g, None)


@pytest.mark.parametrize("shape", BF16_SHAPES)
def test_shape_dense_and_moe(env, shape_env, shape):
    torch, dev, tm = env
    if shape not in GATEUP_TOO_BIG:
        shape_env("gateup", shape)
    shape_env("down", shape)
    w = custom_workload(name="shape_dense", kind="dense", N=777, H=320, I=448, E=1, k=1,
                        coef=0.0, dtype="bf16", seed=11)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"ffn_swiglu_fwd shape {shape} N=777 H=320 I=448")
    y = run_dense(tm, to_dev(inp, dev))
    torch.cuda.synchronize()
    assert rel_l2_per_token(y_to_f64(y), ref["y"]) <= TOL_Y["bf16"]

    w = custom_workload(name="shape_moe", N=1500, H=256, I=320, E=6, k=2, coef=0.01,
                        dtype="bf16", seed=12)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"moe_ffn_fwd shape {shape} N=1500 H=256 I=320 E=6 k=2")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    check_routing(out, ref, w.k, w.E)
    assert rel_l2_per_token(y_to_f64(out.y), ref["y"]) <= TOL_Y["bf16"]


# backward kinds: (override variable, shapes instantiated and valid for it)
BWD_SHAPES = [("bwd_gu", s) for s in
              ("256x128x4x2x128x2", "128x128x2x4x128x2", "256x64x4x2x128x2")] + \
             [("bwd_dh", s) for s in ("128x128x2x4x128x3", "128x128x2x4x128x2")] + \
             [("wgrad_gu", s) for s in
              ("128x256x2x4x128x2", "128x128x2x4x128x3", "128x128x2x2x128x3", "64x64x2x2x128x3")] + \
             [("wgrad_d", s) for s in
              ("128x256x2x4x128x2", "128x128x2x4x128x3", "256x128x4x2x128x3", "128x128x2x2x128x3",
               "64x64x2x2x128x3")]


@pytest.mark.parametrize("var,shape", BWD_SHAPES)
def test_bwd_shape(env, shape_env, var, shape):
    """Each backward launch shape, forced through its override, on a MoE
    backward with ragged tails against the oracle's gradients."""
    import numpy as np

    from oracle.cases import expected_bwd
    from workloads import make_upstream
    from gpu_util import TOL_GRAD, arr_to_dev, rel_l2_per_matrix

    torch, dev, tm = env
    shape_env(var, shape)
    w = custom_workload(name="shape_bwd", N=700, H=192, I=320, E=5, k=2, coef=0.01, dtype="bf16",
                        seed=13)
    inp = make_case(w)
    dy = make_upstream(inp)
    ref = expected_bwd(w, inp, dy)
    announce(f"moe_ffn_bwd {var}={shape} N=700 H=192 I=320 E=5 k=2")
    d = to_dev(inp, dev)
    g = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], arr_to_dev(dy, "bf16", dev),
                       w.k, w.coef)
    torch.cuda.synchronize()
    assert rel_l2_per_token(y_to_f64(g.dx), ref["dx"]) <= TOL_GRAD["bf16"]
    for n in ("dWg", "dWu", "dWd"):
        err = rel_l2_per_matrix(getattr(g, n).double().cpu().numpy(), ref[n])
        assert err <= TOL_GRAD["bf16"], (n, err)
