"""A capacity that drops nothing (capacity factor E: C = N*k >= N) takes the
capacity path -- the permutation kernel with keep flags, the down GEMM into
slots, the combine over kept slots -- and must give the dropless y bit for
bit (the same groups, the same slot values, the same fixed-order sum); both
against the oracle, and repeated calls on one workspace give the same bits."""
import numpy as np
import pytest

from oracle import moe_ffn
from oracle.cases import custom_workload, make_case, widen
from gpu_util import TOL_Y, announce, rel_l2_per_token, to_dev, torch_dev, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


CASES = [  # N, H, I, E, k, dtype, residual
    (32, 2048, 1408, 16, 2, "bf16", True),     # decode: in-block routing
    (700, 256, 512, 8, 2, "bf16", False),
    (1200, 512, 768, 8, 2, "bf16", True),      # 256-row tiles
    (300, 192, 320, 6, 3, "bf16", True),
    (257, 128, 256, 5, 2, "fp32", True),
    (90, 128, 192, 4, 4, "fp32", False),       # k = E
]


@pytest.mark.parametrize("N,H,I,E,k,dt,res", CASES)
def test_capacity_without_drops_is_dropless(env, N, H, I, E, k, dt, res):
    torch, dev, tm = env
    w = custom_workload(name="fc", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt, residual=res,
                        seed=3 * N + k)
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef, residual=f.get("residual"))
    d = to_dev(inp, dev)
    announce(f"capacity without drops N={N} H={H} I={I} E={E} k={k} {dt} residual={res}")
    tdt = d["x"].dtype
    ws = torch.empty(tm.moe_workspace_bytes(N, H, I, E, k, tdt), dtype=torch.uint8, device=dev)
    run = lambda cf: tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef,
                                    residual=d.get("residual"), capacity_factor=cf,
                                    workspace=ws).y.clone()
    y_dropless = run(0.0)
    y_again = run(0.0)
    y_capacity = run(float(E))    # capacity N*k: nothing dropped
    torch.cuda.synchronize()
    view = torch.int16 if tdt == torch.bfloat16 else torch.int32
    assert torch.equal(y_dropless.view(view), y_again.view(view))
    assert torch.equal(y_dropless.view(view), y_capacity.view(view))
    err = rel_l2_per_token(y_to_f64(y_dropless), ref["y"])
    assert err <= TOL_Y[dt], err
