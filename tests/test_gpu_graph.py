"""The entry points under HIP graph capture (torch.cuda.graph): no allocation,
memset or host synchronisation inside, so a captured forward or backward
replays to the same bits as the eager call.  Each graph is replayed several
times with eager work of the program (another call of the same entry point on
other inputs, a library reduction, synchronisations) between the replays, and
every replay is checked against the eager result."""
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


def same(torch, a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def replay_checks(torch, dev, graph, outs, want, other_call):
    for r in range(3):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, o in zip(want, outs):
            assert same(torch, o, want[name]), (r, name)
        other_call()  # eager work between the replays
        torch.randn(1 << 16, device=dev).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("N,H,I,E,k,fused_router", [
    (600, 128, 192, 8, 2, 0),
    (32, 2048, 1408, 16, 2, 1),   # decode-sized: router and grouping inside the GEMM launches
])
def test_graph_moe_forward(env, N, H, I, E, k, fused_router):
    torch, dev, tm = env
    from top_moe_layer_amd import _binding as B

    assert B.moe_fwd_path(N, H, I, E, k, B.DTYPE_BF16)["router_in_up"] == fused_router
    w = custom_workload(name="graph_moe", N=N, H=H, I=I, E=E, k=k, coef=0.01, seed=31)
    d = to_dev(make_case(w), dev)
    d2 = to_dev(make_case(custom_workload(name="graph_moe2", N=N, H=H, I=I, E=E, k=k,
                                          coef=0.01, seed=32)), dev)
    N, H, E, k = w.N, w.H, w.E, w.k
    ws = torch.empty(tm.moe_workspace_bytes(N, H, w.I, E, k, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    alpha = torch.empty((N, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)

    def call(src, stream=None):
        tm.moe_ffn_fwd(src["x"], src["Wr"], src["Wg"], src["Wu"], src["Wd"], k, w.coef, y=y,
                       topk_idx=idx, alpha=alpha, aux_loss=aux, expert_offsets=offs,
                       return_lists=False, workspace=ws, stream=stream)

    announce(f"graph capture of moe_ffn_fwd N={N} H={H} I={I} E={E} k={k}")
    call(d)
    torch.cuda.synchronize()
    want = {"y": y.clone(), "idx": idx.clone(), "alpha": alpha.clone(), "aux": aux.clone(),
            "offs": offs.clone()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(d, torch.cuda.current_stream())
    replay_checks(torch, dev, g, [y, idx, alpha, aux, offs], want, lambda: call(d2))


def test_graph_dense_forward(env):
    torch, dev, tm = env
    w = custom_workload(name="graph_dense", kind="dense", N=300, H=128, I=256, E=1, k=1,
                        coef=0.0, seed=33)
    d = to_dev(make_case(w), dev)
    ws = torch.empty(tm.ffn_workspace_bytes(w.N, w.H, w.I, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)
    x2 = torch.randn_like(d["x"].float()).to(torch.bfloat16)

    def call(x, stream=None):
        tm.ffn_swiglu_fwd(x, d["Wg"], d["Wu"], d["Wd"], y=y, workspace=ws, stream=stream)

    announce("graph capture of ffn_swiglu_fwd N=300")
    call(d["x"])
    torch.cuda.synchronize()
    want = {"y": y.clone()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(d["x"], torch.cuda.current_stream())
    replay_checks(torch, dev, g, [y], want, lambda: call(x2))


def test_graph_moe_backward(env):
    torch, dev, tm = env
    w = custom_workload(name="graph_moe_bwd", N=300, H=128, I=128, E=8, k=2, coef=0.01, seed=34)
    inp = make_case(w)
    d = to_dev(inp, dev)
    dy = arr_to_dev(make_upstream(inp), "bf16", dev)
    dy2 = torch.randn_like(dy.float()).to(torch.bfloat16)
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    ws = torch.empty(tm.moe_bwd_workspace_bytes(N, H, I, E, k, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    names = ("dx", "dWr", "dWg", "dWu", "dWd")

    def call(g_in, stream=None):
        return tm.moe_ffn_bwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], g_in, k, w.coef,
                              workspace=ws, stream=stream)

    announce("graph capture of moe_ffn_bwd N=300 E=8 k=2")
    eager = call(dy)
    torch.cuda.synchronize()
    want = {n: getattr(eager, n).clone() for n in names}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = call(dy, torch.cuda.current_stream())  # the graph's own output tensors
    replay_checks(torch, dev, g, [getattr(captured, n) for n in names], want, lambda: call(dy2))


def test_graph_moe_train_step(env):
    """The training step (forward keeping g, u, then the backward taking them)
    captured as one graph; the eager work between replays runs the same step on
    other inputs through the same saved buffer."""
    torch, dev, tm = env
    w = custom_workload(name="graph_moe_train", N=400, H=128, I=192, E=8, k=2, coef=0.01,
                        seed=35)
    inp = make_case(w)
    d = to_dev(inp, dev)
    d2 = to_dev(make_case(custom_workload(name="graph_moe_train2", N=400, H=128, I=192, E=8,
                                          k=2, coef=0.01, seed=36)), dev)
    dy = arr_to_dev(make_upstream(inp), "bf16", dev)
    N, H, I, E, k = w.N, w.H, w.I, w.E, w.k
    ws = torch.empty(tm.moe_workspace_bytes(N, H, I, E, k, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    saved = torch.empty(tm.moe_bwd_workspace_bytes(N, H, I, E, k, torch.bfloat16),
                        dtype=torch.uint8, device=dev)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    names = ("dx", "dWr", "dWg", "dWu", "dWd")

    def step(src, stream=None):
        tm.moe_ffn_fwd(src["x"], src["Wr"], src["Wg"], src["Wu"], src["Wd"], k, w.coef, y=y,
                       return_lists=False, workspace=ws, saved=saved, stream=stream)
        return tm.moe_ffn_bwd(src["x"], src["Wr"], src["Wg"], src["Wu"], src["Wd"], dy, k,
                              w.coef, workspace=saved, from_saved=True, stream=stream)

    announce("graph capture of the training step N=400 E=8 k=2")
    eager = step(d)
    torch.cuda.synchronize()
    want = {n: getattr(eager, n).clone() for n in names}
    want["y"] = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step(d, torch.cuda.current_stream())
    outs = [getattr(captured, n) for n in names] + [y]
    replay_checks(torch, dev, g, outs, {**{n: want[n] for n in names}, "y": want["y"]},
                  lambda: step(d2))
