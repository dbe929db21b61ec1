"""GPU checks of the training path that keeps g, u for the backward: the
training forwards (ffn_swiglu_fwd_train, moe_ffn_fwd_train) must give the
same bits as the plain forwards in every output, and a backward that takes
g, u (and, for the MoE, the routing) from the saved buffer
(ffn_swiglu_bwd_saved, moe_ffn_bwd with TOPMOE_MOE_BWD_SAVED) the same bits as
the backward that recomputes them.
The plain paths are checked against the oracle by the parity tests, so
bit-equality carries their parity over.  The saved buffer starts filled with
0xFF bytes (NaN in either dtype), so that any part of it the backward reads
without the forward having written it shows up.
"""
import numpy as np
import pytest

from oracle.cases import custom_workload, make_case
from workloads import make_upstream
from gpu_util import announce, arr_to_dev, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def same(torch, a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    assert a.shape == b.shape and a.dtype == b.dtype, what
    av = a.contiguous().view(-1).view(torch.uint8) if a.numel() else a
    bv = b.contiguous().view(-1).view(torch.uint8) if b.numel() else b
    assert torch.equal(av, bv), f"{what}: not bit-identical"


def garbage(torch, nbytes, dev):
    return torch.full((max(nbytes, 256),), 255, dtype=torch.uint8, device=dev)


DENSE = [
    # N, H, I, dtype, residual
    (100, 768, 2432, "fp32", False),   # the small dense case
    (300, 256, 512, "bf16", True),     # ragged rows, residual
    (1000, 512, 1408, "bf16", False),
    (64, 128, 192, "fp32", True),
    (0, 128, 128, "bf16", False),      # empty
]


@pytest.mark.parametrize("N,H,I,dt,res", DENSE)
def test_dense_train_forward_and_saved_backward(env, N, H, I, dt, res):
    torch, dev, tm = env
    w = custom_workload(name=f"tr_{N}_{H}_{I}", kind="dense", N=max(N, 1), H=H, I=I, E=1, k=1,
                        dtype=dt, residual=res, seed=N + H + I)
    inp = make_case(w, N=N)
    d = to_dev(inp, dev)
    dy = arr_to_dev(make_upstream(inp), dt, dev)
    tdt = d["x"].dtype
    announce(f"dense train fwd / saved bwd N={N} H={H} I={I} {dt} residual={res}")
    y0 = tm.ffn_swiglu_fwd(d["x"], d["Wg"], d["Wu"], d["Wd"], residual=d.get("residual"))
    saved = garbage(torch, tm.ffn_bwd_workspace_bytes(N, H, I, tdt), dev)
    y1 = tm.ffn_swiglu_fwd(d["x"], d["Wg"], d["Wu"], d["Wd"], residual=d.get("residual"),
                           saved=saved)
    g0 = tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], dy)
    g1 = tm.ffn_swiglu_bwd(d["x"], d["Wg"], d["Wu"], d["Wd"], dy, workspace=saved,
                           from_saved=True)
    torch.cuda.synchronize()
    same(torch, y0, y1, "y")
    for n in ("dx", "dWg", "dWu", "dWd"):
        same(torch, getattr(g0, n), getattr(g1, n), n)
    if N:
        assert torch.isfinite(g1.dWd.float()).all()


MOE = [
    # N, H, I, E, k, z_coef, capacity_factor, norm_topk_prob, residual, dtype
    (4096, 768, 2432, 4, 1, 0.0, 0.0, True, False, "bf16"),    # the top-1 workload's shape
    (300, 128, 192, 8, 2, 0.0, 0.0, True, False, "bf16"),
    (257, 64, 128, 4, 1, 0.002, 0.8, True, True, "bf16"),      # z-loss, capacity, residual
    (300, 128, 128, 8, 2, 0.001, 1.0, False, False, "bf16"),   # raw top-k weights, capacity
    (200, 64, 64, 4, 2, 0.01, 0.5, True, True, "fp32"),
    (96, 128, 128, 16, 4, 0.0, 0.0, True, False, "fp32"),      # experts with no tokens
    (0, 64, 64, 4, 2, 0.0, 0.0, True, False, "bf16"),          # empty
]


@pytest.mark.parametrize("N,H,I,E,k,zc,cf,norm,res,dt", MOE)
def test_moe_train_forward_and_saved_backward(env, N, H, I, E, k, zc, cf, norm, res, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"trm_{N}_{E}_{k}", N=max(N, 1), H=H, I=I, E=E, k=k, coef=0.01,
                        dtype=dt, residual=res, seed=3 * N + E + k)
    inp = make_case(w, N=N)
    d = to_dev(inp, dev)
    dy = arr_to_dev(make_upstream(inp), dt, dev)
    tdt = d["x"].dtype
    kw = dict(residual=d.get("residual"), z_coef=zc, capacity_factor=cf, norm_topk_prob=norm)
    announce(f"moe train fwd / saved bwd N={N} H={H} I={I} E={E} k={k} z={zc} cap={cf} "
             f"norm={norm} {dt}")
    o0 = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, 0.01, **kw)
    saved = garbage(torch, tm.moe_bwd_workspace_bytes(N, H, I, E, k, tdt), dev)
    o1 = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, 0.01, saved=saved, **kw)
    bkw = dict(z_coef=zc, capacity_factor=cf, norm_topk_prob=norm, aux_grad=0.5, z_grad=2.0)
    g0 = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dy, k, 0.01, **bkw)
    g1 = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dy, k, 0.01, **bkw,
                        workspace=saved, from_saved=True)
    torch.cuda.synchronize()
    for n in ("y", "topk_idx", "alpha", "aux_loss", "z_loss", "expert_offsets",
              "sorted_token_ids"):
        same(torch, getattr(o0, n), getattr(o1, n), n)
    for n in ("dx", "dWr", "dWg", "dWu", "dWd"):
        same(torch, getattr(g0, n), getattr(g1, n), n)
    if N:
        assert torch.isfinite(g1.dWd.float()).all() and torch.isfinite(g1.dWr).all()


def test_saved_buffer_reused_across_steps(env):
    """Two training steps on different inputs through one saved buffer: the
    second step's backward sees only the second forward's g, u."""
    torch, dev, tm = env
    N, H, I, E, k = 500, 128, 256, 8, 2
    saved = garbage(torch, tm.moe_bwd_workspace_bytes(N, H, I, E, k, torch.bfloat16), dev)
    for seed in (11, 12):
        w = custom_workload(name=f"reuse_{seed}", N=N, H=H, I=I, E=E, k=k, coef=0.01,
                            dtype="bf16", seed=seed)
        inp = make_case(w)
        d = to_dev(inp, dev)
        dy = arr_to_dev(make_upstream(inp), "bf16", dev)
        announce(f"saved buffer reuse, step seed {seed}")
        tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, 0.01, saved=saved)
        g1 = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dy, k, 0.01,
                            workspace=saved, from_saved=True)
        g0 = tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], dy, k, 0.01)
        torch.cuda.synchronize()
        for n in ("dx", "dWr", "dWg", "dWu", "dWd"):
            same(torch, getattr(g0, n), getattr(g1, n), n)


@pytest.mark.parametrize("kind", ["dense", "moe"])
def test_autograd_keep_activations(env, kind):
    """The autograd Functions give the same gradients whether the forward keeps
    g, u (the default) or the backward recomputes them."""
    torch, dev, tm = env
    if kind == "dense":
        w = custom_workload(name="ag_dense", kind="dense", N=260, H=256, I=384, E=1, k=1,
                            dtype="bf16", seed=5)
    else:
        w = custom_workload(name="ag_moe", N=260, H=256, I=384, E=8, k=2, coef=0.01,
                            dtype="bf16", seed=6)
    inp = make_case(w)
    d = to_dev(inp, dev)
    dy = arr_to_dev(make_upstream(inp), "bf16", dev)
    announce(f"autograd keep_activations {kind}")
    grads = []
    for keep in (True, False):
        leaves = {n: t.clone().requires_grad_(True) for n, t in d.items() if n != "residual"}
        if kind == "dense":
            y = tm.swiglu_ffn(leaves["x"], leaves["Wg"], leaves["Wu"], leaves["Wd"],
                              keep_activations=keep)
            loss = (y.float() * dy.float()).sum()
        else:
            y, aux, z, _, _ = tm.moe_ffn(leaves["x"], leaves["Wr"], leaves["Wg"], leaves["Wu"],
                                         leaves["Wd"], 2, 0.01, z_coef=0.001,
                                         keep_activations=keep)
            loss = (y.float() * dy.float()).sum() + aux.sum() + z.sum()
        loss.backward()
        grads.append({n: t.grad for n, t in leaves.items()})
    torch.cuda.synchronize()
    for n in grads[0]:
        same(torch, grads[0][n], grads[1][n], n)
