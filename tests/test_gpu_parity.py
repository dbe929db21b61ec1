"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.

Bars: topk_idx, expert offsets and per-expert token lists bit-exact (inputs
drawn with a top-k margin of 1e-3); alpha and aux_loss within 1e-5 relative;
y within a max per-token relative L2 error of 1e-5 (fp32 path) or 2e-2 (bf16
inputs, fp32 accumulation).  Small shapes are checked in full; the workloads
at their full sizes are checked on every routing output and on sampled rows
of y, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from oracle.cases import custom_workload, expected, make_case
from workloads import get
from gpu_util import (TOL_Y, announce, check_routing, rel_l2_global, rel_l2_per_token,
                      run_dense, run_moe, sample_rows, to_dev, torch_dev, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


# ------------------------------------------------------------------ dense
DENSE_SMALL = [
    (1, 64, 64), (7, 128, 192), (129, 64, 128), (300, 128, 64), (513, 192, 320), (1000, 256, 448),
]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,H,I", DENSE_SMALL)
def test_dense_small(env, N, H, I, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"dense_{N}_{H}_{I}", kind="dense", N=N, H=H, I=I, E=1, k=1,
                        coef=0.0, dtype=dt, seed=N + H + I)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"ffn_swiglu_fwd N={N} H={H} I={I} {dt}")
    y = run_dense(tm, to_dev(inp, dev))
    torch.cuda.synchronize()
    err = rel_l2_per_token(y_to_f64(y), ref["y"])
    assert err <= TOL_Y[dt], err


# -------------------------------------------------------------------- moe
MOE_SMALL = [
    # N, H, I, E, k
    (1, 64, 64, 4, 1),
    (7, 64, 128, 2, 2),
    (129, 128, 64, 3, 1),
    (1000, 64, 64, 8, 2),
    (257, 128, 192, 64, 2),
    (100, 64, 64, 1, 1),
    (500, 128, 128, 16, 4),
    (2000, 64, 128, 5, 3),
    # router layouts: W_router in LDS with long rows (H = 2048, and 4096 at the
    # 64 KB limit), and the H-split layout with many tokens (W_router 128 KB)
    # or many experts with long rows
    (600, 2048, 128, 8, 2),
    (300, 4096, 64, 4, 1),
    (300, 2048, 64, 16, 2),
    (20, 4096, 64, 32, 2),
]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,H,I,E,k", MOE_SMALL)
def test_moe_small(env, N, H, I, E, k, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"moe_{N}_{E}_{k}", N=N, H=H, I=I, E=E, k=k, coef=0.01, dtype=dt,
                        seed=N * 7 + E + k)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"moe_ffn_fwd N={N} H={H} I={I} E={E} k={k} {dt}")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    check_routing(out, ref, k, E)
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y[dt], err


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,E", [(64, 8), (33, 3), (40, 64)])
def test_moe_k_equals_E(env, N, E, dt):
    """k = E selects every expert (no margin needed); slots compared by id."""
    torch, dev, tm = env
    w = custom_workload(name=f"moe_kE_{N}_{E}", N=N, H=64, I=64, E=E, k=E, coef=0.01, dtype=dt,
                        seed=3 * N + E)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"moe_ffn_fwd k=E N={N} E={E} {dt}")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    check_routing(out, ref, E, E, exact_order=False)
    assert rel_l2_per_token(y_to_f64(out.y), ref["y"]) <= TOL_Y[dt]


# Decode-sized calls: a few rows per expert, some experts empty, and with a
# skewed router (bias_std / bias_scale shift the logits) one expert holding
# many of the rows.
DECODE_CASES = [
    # N, H, I, E, k, bias_scale
    (1, 128, 192, 8, 2, 0.0),
    (30, 256, 128, 8, 2, 0.0),
    (32, 256, 128, 16, 2, 1.0),
    (5, 64, 64, 1, 1, 0.0),
]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,H,I,E,k,bias", DECODE_CASES)
def test_moe_decode_sized(env, N, H, I, E, k, bias, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"moe_decode_{N}_{E}_{k}", N=N, H=H, I=I, E=E, k=k, coef=0.01,
                        dtype=dt, bias_std=1.5 if bias else 0.0, bias_scale=bias, seed=N + 3 * E)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"moe_ffn_fwd (decode-sized) N={N} H={H} I={I} E={E} k={k} {dt}")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    check_routing(out, ref, w.k, w.E)
    assert rel_l2_per_token(y_to_f64(out.y), ref["y"]) <= TOL_Y[dt]


# Block context (lesson 13, sections 1.3-1.4: hidden_states + mlp(...)) and
# norm_topk_prob False (walkthrough step 5): the residual stream is added to y
# before its single rounding, also when y is the residual tensor itself.
BLOCK_CASES = [
    # kind, N, H, I, E, k, residual, norm, in_place
    ("dense", 300, 128, 192, 1, 1, True, True, False),
    ("dense", 5, 64, 128, 1, 1, True, True, True),
    ("moe", 700, 128, 128, 8, 1, True, True, False),
    ("moe", 700, 128, 128, 8, 2, True, True, True),
    ("moe", 700, 128, 128, 8, 2, False, False, False),
    ("moe", 33, 256, 64, 16, 3, True, False, True),
    ("moe", 1500, 64, 128, 4, 1, False, False, False),
]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("kind,N,H,I,E,k,res,norm,in_place", BLOCK_CASES)
def test_block_context(env, kind, N, H, I, E, k, res, norm, in_place, dt):
    torch, dev, tm = env
    w = custom_workload(name=f"block_{kind}_{N}_{E}_{k}", kind=kind, N=N, H=H, I=I, E=E, k=k,
                        coef=0.01 if kind == "moe" else 0.0, dtype=dt, residual=res,
                        norm_topk_prob=norm, seed=N + 5 * E + k)
    inp = make_case(w)
    ref = expected(w, inp)
    announce(f"{kind} residual={res} norm_topk_prob={norm} in_place={in_place} N={N} E={E} k={k} {dt}")
    d = to_dev(inp, dev)
    y = d["residual"] if in_place else None
    if kind == "dense":
        out_y = run_dense(tm, d, y=y)
    else:
        out = run_moe(tm, d, w, y=y)
        out_y = out.y
        check_routing(out, ref, w.k, w.E)
    torch.cuda.synchronize()
    if in_place:
        assert out_y.data_ptr() == d["residual"].data_ptr()
    assert rel_l2_per_token(y_to_f64(out_y), ref["y"]) <= TOL_Y[dt]


def test_moe_top1_alpha_exactly_one(env):
    torch, dev, tm = env
    w = custom_workload(name="moe_alpha1", N=777, H=128, I=64, E=8, k=1, coef=0.01, seed=5)
    inp = make_case(w)
    announce("moe_ffn_fwd k=1 alpha == 1")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    assert bool((out.alpha == 1.0).all())


def test_moe_coef_zero_gives_zero_aux(env):
    torch, dev, tm = env
    w = custom_workload(name="moe_coef0", N=300, H=64, I=64, E=4, k=2, coef=0.0, seed=6)
    inp = make_case(w)
    announce("moe_ffn_fwd coef=0")
    out = run_moe(tm, to_dev(inp, dev), w)
    torch.cuda.synchronize()
    assert float(out.aux_loss.cpu()[0]) == 0.0


def test_moe_single_expert_matches_dense(env):
    """E = 1, k = 1 reduces the MoE to the dense FFN (both against the oracle)."""
    torch, dev, tm = env
    w = custom_workload(name="moe_e1", N=300, H=128, I=192, E=1, k=1, coef=0.01, seed=8)
    inp = make_case(w)
    ref = expected(w, inp)
    d = to_dev(inp, dev)
    announce("moe_ffn_fwd E=1 vs ffn_swiglu_fwd")
    out = run_moe(tm, d, w)
    yd = tm.ffn_swiglu_fwd(d["x"], d["Wg"][0], d["Wu"][0], d["Wd"][0])
    torch.cuda.synchronize()
    assert rel_l2_per_token(y_to_f64(out.y), ref["y"]) <= TOL_Y["bf16"]
    assert rel_l2_per_token(y_to_f64(yd), ref["y"]) <= TOL_Y["bf16"]


def test_moe_eval_flag(env):
    """Outside training the module's aux loss is a zero scalar ([L13] step 6);
    everything else is the training-mode result, bit for bit."""
    torch, dev, tm = env
    w = custom_workload(name="moe_eval", N=300, H=128, I=128, E=8, k=2, coef=0.01, seed=31)
    d = to_dev(make_case(w), dev)
    announce("moe_ffn_fwd training=False")
    a = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef, z_coef=0.01)
    b = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef, z_coef=0.01,
                       training=False)
    torch.cuda.synchronize()
    assert float(a.aux_loss.cpu()[0]) > 0 and float(a.z_loss.cpu()[0]) > 0
    assert float(b.aux_loss.cpu()[0]) == 0.0 and float(b.z_loss.cpu()[0]) == 0.0
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))
    assert torch.equal(a.topk_idx, b.topk_idx) and torch.equal(a.alpha, b.alpha)


def test_moe_on_a_side_stream(env):
    """A call on a stream other than the current one allocates its outputs and
    workspace for that stream and gives the same bits."""
    torch, dev, tm = env
    w = custom_workload(name="moe_side", N=700, H=128, I=192, E=8, k=2, coef=0.01, seed=32)
    d = to_dev(make_case(w), dev)
    announce("moe_ffn_fwd on a side stream")
    ref = run_moe(tm, d, w)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef, stream=side)
    junk = torch.full((1 << 22,), 7, dtype=torch.int32, device=dev)  # current-stream traffic
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out.y.view(torch.int16), ref.y.view(torch.int16))
    assert torch.equal(out.sorted_token_ids, ref.sorted_token_ids)


def test_empty_inputs(env):
    torch, dev, tm = env
    announce("N = 0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    Wr = torch.zeros((4, 64), dtype=torch.float32, device=dev)
    out = tm.moe_ffn_fwd(x, Wr, W, W, W, 2, 0.01)
    y = tm.ffn_swiglu_fwd(x, W[0], W[0], W[0])
    torch.cuda.synchronize()
    assert out.y.shape == (0, 64) and y.shape == (0, 64)
    assert out.expert_offsets.cpu().tolist() == [0] * 5
    assert float(out.aux_loss.cpu()[0]) == 0.0


def test_bitwise_deterministic(env):
    torch, dev, tm = env
    w = custom_workload(name="moe_det", N=3000, H=128, I=192, E=8, k=2, coef=0.01, seed=9)
    inp = make_case(w)
    d = to_dev(inp, dev)
    announce("moe_ffn_fwd run-to-run determinism")
    a = run_moe(tm, d, w)
    b = run_moe(tm, d, w)
    torch.cuda.synchronize()
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))
    assert torch.equal(a.alpha, b.alpha) and torch.equal(a.aux_loss, b.aux_loss)
    assert torch.equal(a.sorted_token_ids, b.sorted_token_ids)


# ------------------------------------------------- workloads at full size
FULL = ["dense_fp32", "moe_top1", "dense_bf16", "moe_skew", "moe_skew_literal", "moe_decode"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size(env, name):
    """Every token row of y against the oracle at the workload's full size, in
    the launch configuration the benchmark times."""
    torch, dev, tm = env
    w = get(name)
    inp = make_case(w)
    announce(f"{w.name}: N={w.N} H={w.H} I={w.I} E={w.E} k={w.k} {w.dtype}: oracle (all rows)")
    ref = expected(w, inp)
    announce(f"{w.name}: GPU")
    d = to_dev(inp, dev)
    if w.kind == "dense":
        y = run_dense(tm, d)
        torch.cuda.synchronize()
    else:
        out = run_moe(tm, d, w)
        torch.cuda.synchronize()
        check_routing(out, ref, w.k, w.E)
        y = out.y
    got = y_to_f64(y)
    assert got.shape == ref["y"].shape
    err = rel_l2_per_token(got, ref["y"])
    print(f"[gpu] {w.name}: max per-token rel L2 {err:.3e}, global {rel_l2_global(got, ref['y']):.3e}",
          flush=True)
    assert err <= TOL_Y[w.dtype], err
